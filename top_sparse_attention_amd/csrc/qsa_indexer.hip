// The QSA indexer and Top-K selection (gfx950): the step that produces the
// selection rows the sparse attention reads.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include "qsa_device.h"
#include "qsa_kernels.h"
#include "qsa_indexer.h"

namespace qsa {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// score[t, c] = sum_h max(0, iq[t,h] . ik[c]) with bf16 MFMA.  A workgroup
// takes 128 tokens (32 per wave, as 8 MFMA row tiles of 4 tokens x 4 heads;
// 64 measured 2% slower, each key tile then read from LDS by twice as many
// waves per token) and one range of kScoreSplit index keys, walked in tiles
// of 64 blocks staged in LDS (swizzled) and shared by all row tiles; it stops at the
// last block any of its tokens may select.  MFMA rows are (token, head)
// pairs, so lane (c, j) of a 16x16 output holds the 4 heads of one token
// against block c and the head sum stays in the lane.  Each tile's 128 x 64
// scores go through LDS and are stored as whole 256-byte row segments.
constexpr int kScoreTokens = 128;
constexpr int kScoreRowTiles = kScoreTokens / 4 / 4;   // per wave
constexpr int kScoreTile = 64;
constexpr int kIndexRowBytes = kIndexDim * 2;   // 256 B
constexpr int kScoreOutPitch = kScoreTile + 4;  // floats per staged row (16-byte aligned)

// Order-preserving map of FP32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t score_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// max(x, 0) for the finite dot products here, as one integer max on the bits
// (negative floats, -0.0 included, are negative integers).  fmaxf costs a
// second instruction per value to quiet a NaN first.
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// Marks, in the first output word, a row that a fast selection left to the
// exact selection on the full row (no output word holds a value below -1).
constexpr int32_t kSelDeferred = INT32_MIN;

// What indexer_scores_kernel writes: every score of the tokens' eligible
// blocks, or only the candidates at or above each token's estimated
// threshold (the fused Top-K), or every score but only where a token's row
// was deferred by the fused selection.
enum ScoreMode { kAllScores, kCandidates, kDeferredRows };

// LDS byte offset of 16-byte chunk `chunk` of index-key tile row `r`.  The
// chunk index is XOR-swizzled by a bijection of r & 7 so that the 8 rows read
// by one phase of a 16-byte read hit 8 different bank groups.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int idx_off(int r, int chunk) {
    return r * kIndexRowBytes + ((chunk ^ swz(r)) << 4);
}

//
// Candidate mode (the fused Top-K): each token keeps, of its eligible blocks
// (4c + 3 <= p), the scores whose key reaches its estimated threshold tau[t],
// as (score, block id) pairs in block order in its row's part for this key
// range: the 16 threads that store a staged row's 64 scores scan their pass
// counts and append at the row's running count.  The count goes to
// counts[t * R + range] at the end (it may exceed the part's room; the
// selection then takes the full row instead).
// kRowStores (every score, rows of a multiple of 4 scores, 16-byte aligned,
// fewer than 2^31 bytes per workgroup's rows): the 16-byte stores are buffer
// stores issued unconditionally, those outside the rows or past the walk
// sent to an offset past the buffer's end, which the hardware drops.  With a
// branch around each store the compiler cannot count the stores issued
// after the next key tile's loads, so its wait for those loads also waited
// for the previous tile's stores.
template <int kMode, bool kRowStores = false>
__global__ __launch_bounds__(256) void indexer_scores_kernel(const IndexerScoreParams p) {
    static_assert(!kRowStores || kMode == kAllScores, "row stores write every score");
    // One key tile: the barrier after each tile's scores also orders its reads
    // before the next tile is written.
    __shared__ __attribute__((aligned(16))) char tile[kScoreTile * kIndexRowBytes];
    __shared__ __attribute__((aligned(16))) float out_tile[kScoreTokens * kScoreOutPitch];
    __shared__ int c_end_shared, any_deferred;
    // Candidate mode: per token of the workgroup its eligible blocks, its
    // threshold key and its running candidate count in this range (in LDS:
    // the MFMA operands already hold most of the registers).
    __shared__ int tok_lim[kMode == kCandidates ? kScoreTokens : 1];
    __shared__ uint32_t tok_tau[kMode == kCandidates ? kScoreTokens : 1];
    __shared__ int seg_cnt[kMode == kCandidates ? kScoreTokens : 1];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, j = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * kScoreTokens;
    const int c_begin = blockIdx.y * kScoreSplit;

    if (tid == 0) {
        c_end_shared = 0;
        any_deferred = 0;
    }
    __syncthreads();
    if (tid < kScoreTokens && t0 + tid < p.T) {
        const int64_t lim = min<int64_t>(max<int64_t>(((int64_t)p.positions[t0 + tid] + 1) /
                                                          kIndexBlock, 0), p.C);
        atomicMax(&c_end_shared, (int)lim);
        if constexpr (kMode == kCandidates) {
            tok_lim[tid] = (int)lim;
            tok_tau[tid] = p.tau[t0 + tid];
            seg_cnt[tid] = 0;
        }
        if constexpr (kMode == kDeferredRows)
            if (p.deferred[(t0 + tid) * p.deferred_stride] == kSelDeferred) any_deferred = 1;
    }
    if (kMode == kCandidates && tid < kScoreTokens && t0 + tid >= p.T) {
        tok_lim[tid] = 0;
        tok_tau[tid] = 0;
        seg_cnt[tid] = 0;
    }
    __syncthreads();
    if (kMode == kDeferredRows && !any_deferred) return;
    const int c_end = min(c_end_shared, c_begin + kScoreSplit);
    if (c_begin >= c_end) {
        if constexpr (kMode == kCandidates)
            if (tid < kScoreTokens && t0 + tid < p.T) p.counts[(t0 + tid) * p.R + blockIdx.y] = 0;
        return;
    }

    // A operands: row tile rt of this wave is tokens t0 + 32 wave + 4 rt ..+3;
    // row r of a tile = (token r/4, head r%4), dims 32 ks + 8 j.
    bf16x8_t qa[kScoreRowTiles][4];
#pragma unroll
    for (int rt = 0; rt < kScoreRowTiles; ++rt) {
        const int64_t ta = t0 + (kScoreTokens / 4) * wave + 4 * rt + (c >> 2);
        const uint16_t *qrow =
            ta < p.T ? p.iq + ta * p.q_st + (int64_t)(c & 3) * p.q_sh : kZeroRow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qa[rt][ks] = ldg16<bf16x8_t>(qrow + 32 * ks + 8 * j);
    }

    // Staging: 64 rows x 16 chunks = 1024 chunks, 4 per thread.
    auto load_tile = [&](int c0, u32x4_t (&r)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + 256 * u;
            const int row = idx >> 4, ch = idx & 15;
            const int64_t blk = c0 + row;
            const uint16_t *src = blk < c_end ? p.ik + blk * p.k_st + ch * 8 : kZeroRow + ch * 8;
            r[u] = ldg16<u32x4_t>(src);
        }
    };
    auto store_tile = [&](char *dst, const u32x4_t (&r)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + 256 * u;
            *LDS_PTR(u32x4_t, dst + idx_off(idx >> 4, idx & 15)) = r[u];
        }
    };
    // The staged scores go out as 16-byte stores where the rows allow it.
    const bool vec_out = (p.C % 4) == 0 && ((uintptr_t)p.scores % 16) == 0;
    // (Unused, and removed, unless kRowStores.)
    const __amdgpu_buffer_rsrc_t rows_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        p.scores + t0 * p.C, (short)0,
        kRowStores ? (int)(min<int64_t>(kScoreTokens, p.T - t0) * p.C * 4) : 0, 0x00020000);

    // The next key tile is loaded during this tile's scores and written to
    // LDS after this tile's scores are stored: its wait then follows those
    // stores in the same iteration (the memory counter retires in issue
    // order, so a wait for loads issued before the stores counts them).
    u32x4_t stage[4];
    load_tile(c_begin, stage);
    store_tile(tile, stage);
    __syncthreads();   // the first key tile is staged
    for (int c0 = c_begin; c0 < c_end; c0 += kScoreTile) {
        const bool more = c0 + kScoreTile < c_end;
        if (more) load_tile(c0 + kScoreTile, stage);
        const char *kt = tile;
#pragma unroll
        for (int ct = 0; ct < kScoreTile / 16; ++ct) {
            bf16x8_t kb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kb[ks] = *LDS_PTR(bf16x8_t, kt + idx_off(16 * ct + c, 4 * ks + j));
            // Several row tiles. MFMA chains at a time, interleaved (k-step
            // outer), so consecutive MFMAs never wait for each other's
            // results; four (two beside the candidate state) keep the registers
            // within two waves per SIMD.
            constexpr int kChains = kMode == kCandidates ? 2 : 4;
#pragma unroll
            for (int rt0 = 0; rt0 < kScoreRowTiles; rt0 += kChains) {
                f32x4_t d[kChains];
#pragma unroll
                for (int i = 0; i < kChains; ++i) d[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int i = 0; i < kChains; ++i)
                        d[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rt0 + i][ks], kb[ks],
                                                                       d[i], 0, 0, 0);
#pragma unroll
                for (int i = 0; i < kChains; ++i) {
                    const float score = relu(d[i][0]) + relu(d[i][1]) + relu(d[i][2]) +
                                        relu(d[i][3]);
                    out_tile[((kScoreTokens / 4) * wave + 4 * (rt0 + i) + j) * kScoreOutPitch +
                             16 * ct + c] = score;
                }
            }
        }
        __syncthreads();   // the tile's scores are complete, its keys read
        // kScoreTokens rows of 64 scores: 16 chunks of 4 per row.
#pragma unroll
        for (int u = 0; u < kScoreTokens * (kScoreTile / 4) / 256; ++u) {
            const int idx = tid + 256 * u;
            const int r = idx >> 4, k4 = 4 * (idx & 15);
            const int64_t t_out = t0 + r;
            const int64_t blk = c0 + k4;
            if constexpr (kMode == kCandidates) {
                // The 16 lanes idx & 15 of row r (one 16-lane row of a wave)
                // append their passing scores in block order: an inclusive
                // scan of the pass counts across the row (DPP row shifts),
                // then the row's total from its last lane (DPP row share).
                const f32x4_t v = *(const f32x4_t *)(out_tile + r * kScoreOutPitch + k4);
                const int lim = min(tok_lim[r], c_end);
                const uint32_t tau = tok_tau[r];
                int pass = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pass |= (blk + e < lim && score_key(v[e]) >= tau) ? (1 << e) : 0;
                const int cnt = __popc(pass);
                int incl = cnt;
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xf, 0xf, true);   // row_shr:1
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xf, 0xf, true);   // row_shr:2
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xf, 0xf, true);   // row_shr:4
                incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xf, 0xf, true);   // row_shr:8
                const int total = __builtin_amdgcn_update_dpp(0, incl, 0x15f, 0xf, 0xf, false);   // row_share:15
                const int base = seg_cnt[r];
                int at = base + incl - cnt;
                if ((lane & 15) == 15) seg_cnt[r] = base + total;
                const int room = min(kScoreSplit, (int)(p.C - c_begin)) / 2;
                f32x2_t *seg = (f32x2_t *)(p.scores + t_out * p.pair_pitch + c_begin);
                // One 8-byte store per passing score, lowest block first.
                for (int bits = pass; bits; bits &= bits - 1, ++at) {
                    const int e = __builtin_ctz(bits);
                    const float x = e == 0 ? v[0] : e == 1 ? v[1] : e == 2 ? v[2] : v[3];
                    if (at < room) seg[at] = f32x2_t{x, __int_as_float((int)blk + e)};
                }
            } else if constexpr (kRowStores) {
                const f32x4_t v = *(const f32x4_t *)(out_tile + r * kScoreOutPitch + k4);
                const uint32_t off = t_out < p.T && blk < c_end
                                         ? (uint32_t)(((int64_t)r * p.C + blk) * 4)
                                         : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rows_rsrc,
                                                       (int)off, 0, 0);
            } else if (t_out < p.T && blk < c_end) {
                const f32x4_t v = *(const f32x4_t *)(out_tile + r * kScoreOutPitch + k4);
                float *dst = p.scores + t_out * p.C + blk;
                if (vec_out && blk + 3 < c_end) {
                    *(f32x4_t *)dst = v;
                } else {
                    for (int e = 0; e < 4 && blk + e < c_end; ++e) dst[e] = v[e];
                }
            }
        }
        if (more) store_tile(tile, stage);
        __syncthreads();   // the next key tile is staged; the scores are read
    }
    if constexpr (kMode == kCandidates) {
        if (tid < kScoreTokens && t0 + tid < p.T)
            p.counts[(t0 + tid) * p.R + blockIdx.y] = seg_cnt[tid];
    }
}

// The threshold estimate of the fused Top-K.  A workgroup takes kEstTokens
// consecutive query tokens and samples kEstRuns runs of 16 consecutive blocks
// spread evenly over [0, n_min), n_min the smallest eligible count among its
// tokens that need an estimate (rows of more than kSelCandSmall eligible
// blocks), so every sample is eligible for every token (the tokens of a
// prefill chunk have nearly the same count).  The sampled scores come from
// bf16 MFMA exactly as in indexer_scores_kernel (rows = (token, head)); each
// wave then finds, for each of its 4 tokens, the top 16 bits of the key
// ranked about target * samples / n from the top (two 8-bit radix passes over
// a per-wave LDS histogram), target = sqrt(budget * kFusedCand) candidates:
// the middle, on a log scale, of the counts the selection takes (budget to
// kFusedCand), so the sampling error (about 1 / sqrt(16) of the count at
// the page's budget) rarely leaves that range.  Taking only the top bits
// rounds the estimate down, which only adds candidates.  tau = 0 (every
// eligible block passes) for rows of at most kSelCandSmall eligible blocks.
constexpr int kEstTokens = 16;                 // 4 MFMA row tiles, one per wave
constexpr int kEstRuns = 16;
constexpr int kEstSamples = kEstRuns * 16;     // 256: one 16-key column tile per run
constexpr int kSelCandSmall = 2048;
constexpr int kFusedCand = 4096;               // candidate room of a fused-path row

__global__ __launch_bounds__(256) void indexer_estimate_kernel(const IndexerEstimateParams p) {
    __shared__ float samp[kEstTokens][kEstSamples];
    __shared__ int hist[4][256];
    __shared__ int sh_nmin;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, j = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * kEstTokens;

    auto eligible = [&](int64_t t) -> int {
        if (t >= p.T) return 0;
        const int64_t pos = p.positions[t];
        if (pos < 0 || pos >= p.L) return 0;
        return (int)min<int64_t>((pos + 1) / kIndexBlock, p.C);
    };
    if (tid == 0) sh_nmin = INT32_MAX;
    __syncthreads();
    if (tid < kEstTokens) {
        const int n = eligible(t0 + tid);
        if (n > kSelCandSmall) atomicMin(&sh_nmin, n);
    }
    __syncthreads();
    const int n_min = sh_nmin;
    if (n_min == INT32_MAX) {   // no row needs an estimate
        if (tid < kEstTokens && t0 + tid < p.T) p.tau[t0 + tid] = 0;
        return;
    }

    // Wave w: tokens t0 + 4w .. +3; lane (c, j) holds rows (token c/4, head c%4)
    // of the A operand and, in the output, token j against column c.
    bf16x8_t qa[4];
    {
        const int64_t ta = t0 + 4 * wave + (c >> 2);
        const uint16_t *qrow = ta < p.T ? p.iq + ta * p.q_st + (int64_t)(c & 3) * p.q_sh : kZeroRow;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qa[ks] = ldg16<bf16x8_t>(qrow + 32 * ks + 8 * j);
    }
#pragma unroll 4
    for (int run = 0; run < kEstRuns; ++run) {
        // n_min > kSelCandSmall keeps the runs distinct and inside [0, n_min).
        const int start = (int)((int64_t)run * (n_min - 16) / (kEstRuns - 1)) & ~15;
        const uint16_t *krow = p.ik + (int64_t)(start + c) * p.k_st;
        bf16x8_t kb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[ks] = ldg16<bf16x8_t>(krow + 32 * ks + 8 * j);
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb[ks], d, 0, 0, 0);
        samp[4 * wave + j][16 * run + c] =
            fmaxf(d[0], 0.f) + fmaxf(d[1], 0.f) + fmaxf(d[2], 0.f) + fmaxf(d[3], 0.f);
    }
    wave_lds_fence();   // the wave reads back only its own tokens' samples

    int *h = hist[wave];
    for (int tk = 0; tk < 4; ++tk) {
        const int64_t t = t0 + 4 * wave + tk;
        if (t >= p.T) break;
        const int n = eligible(t);
        if (n <= kSelCandSmall) {
            if (lane == 0) p.tau[t] = 0;
            continue;
        }
        const float target = sqrtf((float)p.budget * (float)kFusedCand);
        const int kth = min(kEstSamples, max(1, (int)ceilf(target * kEstSamples / (float)n)));
        uint32_t key[kEstSamples / 64];
#pragma unroll
        for (int i = 0; i < kEstSamples / 64; ++i) key[i] = score_key(samp[4 * wave + tk][lane + 64 * i]);
        uint32_t prefix = 0;
        int need = kth;
        for (int pass = 0; pass < 2; ++pass) {
            const int shift = 24 - 8 * pass;
#pragma unroll
            for (int i = 0; i < 4; ++i) h[4 * lane + i] = 0;
            wave_lds_fence();
#pragma unroll
            for (int i = 0; i < kEstSamples / 64; ++i)
                if (pass == 0 || (key[i] >> 24) == (prefix >> 24))
                    atomicAdd(&h[(key[i] >> shift) & 255], 1);
            wave_lds_fence();
            // lane l owns digits 4l .. 4l + 3; counts of the digits above.
            const int cnt = h[4 * lane] + h[4 * lane + 1] + h[4 * lane + 2] + h[4 * lane + 3];
            int incl = cnt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_down(incl, off);
                if (lane + off < 64) incl += v;
            }
            const int above = incl - cnt;
            const bool mine = above < need && need <= incl;
            int d = 4 * lane + 3, cum = above;
            if (mine)
                while (cum + h[d] < need) cum += h[d--];
            const uint64_t who = __ballot(mine);
            const int src = who ? __builtin_ctzll(who) : 0;
            const int digit = __builtin_amdgcn_readlane(d, src);
            need -= __builtin_amdgcn_readlane(cum, src);
            prefix |= (uint32_t)digit << shift;
            wave_lds_fence();   // the histogram is rewritten by the next pass
        }
        if (lane == 0) p.tau[t] = prefix;
    }
}

// Exclusive prefix sum of x over the 256 threads of a workgroup, in thread
// order, and the workgroup's total: a 64-lane scan per wave, then the four
// wave sums through LDS (wave_sums, 4 ints).  Every thread calls it; it
// returns with the workgroup in step, so wave_sums may be reused at once.
__device__ __forceinline__ int block_exclusive_sum(int x, int *total, int *wave_sums) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
    }
    if (lane == 63) wave_sums[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int c = wave_sums[w];
        before += w < wave ? c : 0;
        all += c;
    }
    __syncthreads();
    *total = all;
    return before + incl - x;
}

// Minimum and maximum of (lo, hi) over the 256 threads of a workgroup, for
// every thread (wave_lo, wave_hi: 4 floats of LDS each).
__device__ __forceinline__ void block_min_max(float *lo, float *hi, float *wave_lo,
                                              float *wave_hi) {
    float a = *lo, b = *hi;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        a = fminf(a, __shfl_xor(a, off));
        b = fmaxf(b, __shfl_xor(b, off));
    }
    if ((threadIdx.x & 63) == 0) {
        wave_lo[threadIdx.x >> 6] = a;
        wave_hi[threadIdx.x >> 6] = b;
    }
    __syncthreads();
    a = fminf(fminf(wave_lo[0], wave_lo[1]), fminf(wave_lo[2], wave_lo[3]));
    b = fmaxf(fmaxf(wave_hi[0], wave_hi[1]), fmaxf(wave_hi[2], wave_hi[3]));
    __syncthreads();
    *lo = a;
    *hi = b;
}


// Find, among the keys of `n` scores that pass `in_set`, the `need`-th largest
// key tau and how many keys equal to tau must be kept (written to sh_prefix /
// sh_need), with 8-bit-digit radix passes.  hist is 256 ints of LDS.  With
// kPasses < 4 only the top 8 * kPasses bits are resolved: the result is the
// need-th largest key with its other bits cleared (a lower bound of it).
template <int kPasses = 4, typename ScoreAt, typename InSet>
__device__ void radix_select(int n, int need, ScoreAt score_at, InSet in_set, int *hist,
                             uint32_t *sh_prefix, int *sh_need) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 32 - 8 * kPasses; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int i0 = 0; i0 < n; i0 += 256) {
            const int i = i0 + tid;
            bool hit = false;
            int digit = 0;
            if (i < n) {
                const float x = score_at(i);
                const uint32_t u = score_key(x);
                hit = in_set(x) && (u & mask) == prefix;
                digit = (u >> shift) & 255;
            }
            // The keys of a row share their leading digits, so most lanes
            // of a wave hit the same bin: the lanes with the first active
            // lane's digit add their count with one atomic.
            const uint64_t active = __ballot(hit);
            if (active) {
                const int lead = __builtin_amdgcn_readlane(digit, __builtin_ctzll(active));
                const uint64_t same = __ballot(hit && digit == lead);
                if (hit && digit == lead) {
                    if ((tid & 63) == __builtin_ctzll(same))
                        atomicAdd(&hist[lead], (int)__popcll(same));
                } else if (hit) {
                    atomicAdd(&hist[digit], 1);
                }
            }
        }
        __syncthreads();
        if (tid < 64) {
            // lane l owns digits 4l..4l+3; suffix sums from the top digit.
            const int cnt = hist[4 * tid] + hist[4 * tid + 1] + hist[4 * tid + 2] + hist[4 * tid + 3];
            int incl = cnt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_down(incl, off);
                if (tid + off < 64) incl += v;
            }
            const int above = incl - cnt;   // keys with higher digits
            if (above < need && need <= incl) {
                int cum = above, d = 4 * tid + 3;
                while (cum + hist[d] < need) cum += hist[d--];
                *sh_prefix = prefix | ((uint32_t)d << shift);
                *sh_need = need - cum;
            }
        }
        __syncthreads();
        prefix = *sh_prefix;
        need = *sh_need;
        mask |= 0xffu << shift;
        __syncthreads();
    }
}

// Per query token: keep the `budget` highest-scoring complete causal blocks
// (ties to the lower block); write their positions in ascending block order,
// the causal tail, slot-mapped, then -1 padding.
//
// select_exact (the whole workgroup, one row of n >= 0 eligible scores)
// writes the kept block ids, in ascending order, at out[4 e] for
// e < min(n, budget); expand_row then turns them into slots.  Its threshold
// is found in two steps: a histogram of 256 buckets that split
// [min, max] of the row linearly (a monotone map, so whole buckets above the
// threshold's bucket are kept and those below dropped), then an exact radix
// select over the keys of that one bucket.  Scores of a row sit in a narrow
// float range, so a radix pass over raw key bits would pile every key into
// one or two bins; the linear buckets spread them.
template <bool kInLds>
__device__ void select_exact(const IndexerSelectParams &p, int n, const float *row, int32_t *out) {
    __shared__ float vals[kInLds ? kSelectLdsBlocks : 1];
    __shared__ int hist[256];
    __shared__ int chunk_gt[256], chunk_eq[256];
    __shared__ int wave_sums[4];
    __shared__ float wave_lo[4], wave_hi[4];
    __shared__ uint32_t sh_prefix;
    __shared__ int sh_need;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Row statistics (and the LDS copy): 16-byte loads, four in flight per
    // thread, so the row arrives in a few memory round trips.
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
    const bool vec_ok = ((uintptr_t)row % 16) == 0;
    const int n4 = vec_ok ? n / 4 : 0;
    for (int base = 0; base < n4; base += 4 * 256) {
        f32x4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i4 = base + u * 256 + tid;
            v[u] = i4 < n4 ? *(const f32x4_t *)(row + 4 * i4)
                           : f32x4_t{lo, lo, lo, lo};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i4 = base + u * 256 + tid;
            if (i4 < n4) {
                if (kInLds) *(f32x4_t *)(vals + 4 * i4) = v[u];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo = fminf(lo, v[u][e]);
                    hi = fmaxf(hi, v[u][e]);
                }
            }
        }
    }
    for (int i = 4 * n4 + tid; i < n; i += 256) {
        const float x = row[i];
        if (kInLds) vals[i] = x;
        lo = fminf(lo, x);
        hi = fmaxf(hi, x);
    }
    auto score_at = [&](int i) -> float { return kInLds ? vals[i] : row[i]; };

    // Threshold key tau and how many keys equal to tau to keep (`need`).
    uint32_t tau = 0;
    int need = n;   // n <= budget: every key (all > 0) is kept
    if (n > p.budget) {
        block_min_max(&lo, &hi, wave_lo, wave_hi);
        const float inv = hi > lo ? 256.0f / (hi - lo) : 0.0f;
        auto bucket = [&](float x) { return min(255, (int)((x - lo) * inv)); };
        // Step 1: the bucket holding the budget-th largest score.
        hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += 256) atomicAdd(&hist[bucket(score_at(i))], 1);
        __syncthreads();
        if (tid < 64) {
            const int cnt = hist[4 * tid] + hist[4 * tid + 1] + hist[4 * tid + 2] + hist[4 * tid + 3];
            int incl = cnt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_down(incl, off);
                if (tid + off < 64) incl += v;
            }
            const int above = incl - cnt;
            if (above < p.budget && p.budget <= incl) {
                int cum = above, d = 4 * tid + 3;
                while (cum + hist[d] < p.budget) cum += hist[d--];
                sh_prefix = (uint32_t)d;
                sh_need = p.budget - cum;
            }
        }
        __syncthreads();
        const int b_star = (int)sh_prefix;
        need = sh_need;
        __syncthreads();
        // Step 2: exact select inside that bucket.
        radix_select(n, need, score_at, [&](float x) { return bucket(x) == b_star; }, hist,
                     &sh_prefix, &sh_need);
        tau = sh_prefix;
        need = sh_need;
    }
    __syncthreads();   // vals written by other threads are read below

    // Keep key > tau, and the first `need` keys == tau in block order.  The
    // row is read in chunks of 64 blocks (one per lane); per-chunk counts are
    // scanned so every kept block knows its output position.  Chunks are
    // handled in groups of 256 (one count per thread).
    int gt_before = 0, eq_before = 0;   // keys > tau / == tau in earlier groups
    const int nchunks = (n + 63) / 64;
    for (int g0 = 0; g0 < nchunks; g0 += 256) {
        const int gn = min(256, nchunks - g0);
        for (int k = wave; k < gn; k += 4) {
            const int i = (g0 + k) * 64 + lane;
            const uint32_t u = i < n ? score_key(score_at(i)) : 0u;
            const uint64_t gt = __ballot(i < n && u > tau);
            const uint64_t eq = __ballot(i < n && u == tau);
            if (lane == 0) {
                chunk_gt[k] = __popcll(gt);
                chunk_eq[k] = __popcll(eq);
            }
        }
        __syncthreads();
        int my_gt = tid < gn ? chunk_gt[tid] : 0, my_eq = tid < gn ? chunk_eq[tid] : 0;
        int gt_tot, eq_tot;
        const int gt_pre = block_exclusive_sum(my_gt, &gt_tot, wave_sums);
        const int eq_pre = block_exclusive_sum(my_eq, &eq_tot, wave_sums);
        if (tid < gn) {
            chunk_gt[tid] = gt_pre;
            chunk_eq[tid] = eq_pre;
        }
        __syncthreads();
        const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
        for (int k = wave; k < gn; k += 4) {
            const int i = (g0 + k) * 64 + lane;
            const uint32_t u = i < n ? score_key(score_at(i)) : 0u;
            const bool is_gt = i < n && u > tau, is_eq = i < n && u == tau;
            const uint64_t eq_mask = __ballot(is_eq);
            const int eq_rank = eq_before + chunk_eq[k] + __popcll(eq_mask & below);
            const bool keep = is_gt || (is_eq && eq_rank < need);
            const uint64_t keep_mask = __ballot(keep);
            const int eq_prior = eq_before + chunk_eq[k];
            // kept before this lane = all keys > tau before it + the first
            // `need` keys == tau before it
            const int w = gt_before + chunk_gt[k] + min(eq_prior, need) +
                          __popcll(keep_mask & below);
            if (keep) out[kIndexBlock * w] = i;   // block id for now, expanded below
        }
        gt_before += gt_tot;
        eq_before += eq_tot;
        __syncthreads();   // chunk counts are rewritten by the next group
    }
}

// Expand every kept block id (written at out[4 e], e < kept) into its 4 slots,
// then write the causal tail and the -1 padding.  All the slot-table reads of
// the row are independent and in flight together.
__device__ void expand_row(const IndexerSelectParams &p, int64_t pos, int kept, int32_t *out,
                           int width) {
    const int tid = threadIdx.x;
    __threadfence_block();
    __syncthreads();
    const bool vec_ok = ((uintptr_t)p.slot_of_pos % 16) == 0 && ((uintptr_t)out % 16) == 0;
    for (int e = tid; e < kept; e += 256) {
        const int64_t blk = out[kIndexBlock * e];
        const int32_t *src = p.slot_of_pos + kIndexBlock * blk;
        if (vec_ok) {
            *(u32x4_t *)(out + kIndexBlock * e) = *(const u32x4_t *)src;
        } else {
            int32_t sl[kIndexBlock];
#pragma unroll
            for (int q = 0; q < kIndexBlock; ++q) sl[q] = src[q];
#pragma unroll
            for (int q = 0; q < kIndexBlock; ++q) out[kIndexBlock * e + q] = sl[q];
        }
    }
    const int r = (int)((pos + 1) % kIndexBlock);
    const int tail0 = kIndexBlock * kept;
    for (int i = tid; i < width - tail0; i += 256)
        out[tail0 + i] = i < r ? p.slot_of_pos[pos - r + 1 + i] : -1;
}


// expand_row for block ids kept in LDS (kept[e], e < n_kept): each thread
// turns its blocks into slots with one 16-byte slot-table load and one
// 16-byte store where aligned.
__device__ void expand_kept(const IndexerSelectParams &p, int64_t pos, int n_kept, const int *kept,
                            int32_t *out, int width) {
    const int tid = threadIdx.x;
    __syncthreads();   // kept[] is complete
    const bool vec_ok = ((uintptr_t)p.slot_of_pos % 16) == 0 && ((uintptr_t)out % 16) == 0;
    for (int e = tid; e < n_kept; e += 256) {
        const int32_t *src = p.slot_of_pos + (int64_t)kIndexBlock * kept[e];
        if (vec_ok) {
            *(u32x4_t *)(out + kIndexBlock * e) = *(const u32x4_t *)src;
        } else {
#pragma unroll
            for (int q = 0; q < kIndexBlock; ++q) out[kIndexBlock * e + q] = src[q];
        }
    }
    const int r = (int)((pos + 1) % kIndexBlock);
    const int tail0 = kIndexBlock * n_kept;
    for (int i = tid; i < width - tail0; i += 256)
        out[tail0 + i] = i < r ? p.slot_of_pos[pos - r + 1 + i] : -1;
}

// kDeferredOnly: a second launch after indexer_select_fast_kernel that
// selects only the rows it deferred (the others return at once).
template <bool kInLds, bool kDeferredOnly = false>
__global__ __launch_bounds__(256) void indexer_select_kernel(const IndexerSelectParams p) {
    const int64_t t = blockIdx.x;
    const int64_t pos = p.positions[t];
    int32_t *out = p.out + t * p.out_stride;
    const int width = kIndexBlock * p.budget + 3;
    if (kDeferredOnly) {
        if (out[0] != kSelDeferred) return;   // the same word for every thread
        __syncthreads();                       // read by all before it is rewritten
    }
    if (pos < 0 || pos >= p.L) {
        for (int i = threadIdx.x; i < width; i += 256) out[i] = -1;
        return;
    }
    const int n = (int)min<int64_t>((pos + 1) / kIndexBlock, p.C);
    select_exact<kInLds>(p, n, p.scores + t * p.C, out);
    expand_row(p, pos, min(n, p.budget), out, width);
}

// The same selection, faster for budgets up to kCand / 4: the threshold
// is first estimated from kSelSample scores in runs spaced evenly over the row (the
// top 16 bits of the key ranked about 2 * budget * kSelSample / n from the
// top); one pass over the row then keeps, in block order, the scores whose
// key is at least the estimate (about 2 * budget of them), and the exact
// selection runs on that short list.  It is exact whenever at least `budget` scores pass the
// estimate (the budget-th largest key and all its ties then pass); rows where
// fewer pass, or more than kCand, take select_exact.  Two sizes: kSelCandSmall
// (budgets up to 512, the page's budget) takes 19.5 KB of LDS and 94
// registers, 5 workgroups per CU, and defers those rows (kDefer: it marks
// them with kSelDeferred and a second launch selects them), since the exact
// selection inlined here would take 4 KB more LDS and 30 more registers;
// kSelCand takes budgets up to 960 at 4 per CU and selects them in place.
// (Held to 64 registers for 8 per CU the small kernel ran twice as slowly.)
constexpr int kSelSample = 1024;
constexpr int kSelCand = 3840;        // multiples of 256
constexpr int kSelPerThread = 16;   // scores per thread per pass over the row
// Candidate i is stored at i + i / 16: the output pass, where thread t reads
// candidates kPer t .. kPer t + kPer - 1, then reads different banks.
__device__ __forceinline__ int cand_at(int i) { return i + (i >> 4); }

// The exact selection among nc candidates (scores cval and block ids cid, in
// block order, candidate i stored at cand_at(i)): the budget-th largest key
// tau and how many keys equal to tau to keep, then the kept block ids in
// block order at kept[e] (LDS, e < budget).  Thread t owns candidates
// [kPer t, kPer (t + 1)); a kept candidate's position is the number of keys
// > tau before it plus the number of kept ties (the first `need` in block
// order) before it.
template <int kCand>
__device__ void select_candidates(int nc, int budget, const float *cval, const int *cid, int *hist,
                                  uint32_t *sh_prefix, int *sh_need, int *wave_sums, int *kept) {
    const int tid = threadIdx.x;
    radix_select(nc, budget, [&](int i) { return cval[cand_at(i)]; }, [](float) { return true; },
                 hist, sh_prefix, sh_need);
    const uint32_t tau = *sh_prefix;
    const int need = *sh_need;
    constexpr int kPer = kCand / 256;
    int gt = 0, eq = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = kPer * tid + k;
        if (i < nc) {
            const uint32_t u = score_key(cval[cand_at(i)]);
            gt += u > tau;
            eq += u == tau;
        }
    }
    // One scan of both counts, packed (each at most kCand < 2^16).
    static_assert(kCand < (1 << 16), "packed counts");
    int total;
    const int both = block_exclusive_sum(gt | (eq << 16), &total, wave_sums);
    int gt_pre = both & 0xffff, eq_pre = both >> 16;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int i = kPer * tid + k;
        if (i < nc) {
            const uint32_t u = score_key(cval[cand_at(i)]);
            if (u > tau) {
                kept[gt_pre + min(eq_pre, need)] = cid[cand_at(i)];
                ++gt_pre;
            } else if (u == tau) {
                if (eq_pre < need) kept[gt_pre + eq_pre] = cid[cand_at(i)];
                ++eq_pre;
            }
        }
    }
}

template <int kCand, int kWavesPerSimd, bool kDefer>
__global__ __launch_bounds__(256, kWavesPerSimd) void indexer_select_fast_kernel(
    const IndexerSelectParams p) {
    static_assert(kCand % 256 == 0 && kCand >= kSelSample, "candidate list");
    // One 16-byte sample load per thread; runs 16 apart or more once n > kCand >= kSelSample.
    static_assert(kSelSample == 4 * 256, "sample runs");
    constexpr int kCandPadded = kCand + kCand / 16;
    __shared__ float cval[kCandPadded];
    __shared__ int cid[kCandPadded];
    __shared__ int kept[kCand / 4];   // budget <= kCand / 4
    __shared__ int hist[256];
    __shared__ int wave_sums[4];
    __shared__ uint32_t sh_prefix;
    __shared__ int sh_need;

    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t pos = p.positions[t];
    int32_t *out = p.out + t * p.out_stride;
    const int width = kIndexBlock * p.budget + 3;
    if (pos < 0 || pos >= p.L) {
        for (int i = tid; i < width; i += 256) out[i] = -1;
        return;
    }
    const int n = (int)min<int64_t>((pos + 1) / kIndexBlock, p.C);
    const float *row = p.scores + t * p.C;
    auto all = [](float) { return true; };

    // Scores [base, base + kSlice) of the row, kSelPerThread consecutive ones
    // per thread (16-byte loads where aligned).
    const bool vec_ok = ((uintptr_t)row % 16) == 0;
    constexpr int kSlice = 256 * kSelPerThread;
    auto load_slice = [&](int base, float (&v)[kSelPerThread]) {
        const int i0 = base + kSelPerThread * tid;
#pragma unroll
        for (int u = 0; u < kSelPerThread / 4; ++u) {
            const int i = i0 + 4 * u;
            if (vec_ok && i + 3 < n) {
                const f32x4_t x = *(const f32x4_t *)(row + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * u + e] = x[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * u + e] = i + e < n ? row[i + e] : 0.0f;
            }
        }
    };

    if (n <= p.budget) {
        for (int e = tid; e < n; e += 256) kept[e] = e;
    } else {
        // The first two slices are in flight while the threshold is estimated.
        float v[kSelPerThread], v1[kSelPerThread];
        load_slice(0, v);
        if (kSlice < n) load_slice(kSlice, v1);
        // 1. Estimated threshold (every key passes when the row fits the list).
        uint32_t tau0 = 0;
        if (n > kCand) {
            // The sample: kSelSample / 16 runs of 16 consecutive scores (64
            // bytes), evenly spaced over the row and aligned to 16 scores.  A
            // strided sample would touch every cache line of the row, which
            // the pass below then fetches a second time.  Thread k loads
            // scores 4 (k % 4) .. + 3 of run k / 4 (n > kCand keeps the runs
            // distinct and inside the row).
            constexpr int kRuns = kSelSample / 16;
            const int start = (int)((int64_t)(tid >> 2) * (n - 16) / (kRuns - 1)) & ~15;
            const int i = start + 4 * (tid & 3);
            f32x4_t x;
            if (vec_ok) {
                x = *(const f32x4_t *)(row + i);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = row[i + e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) cval[4 * tid + e] = x[e];
            __syncthreads();
            const int kth =
                (int)min<int64_t>(kSelSample, (2 * (int64_t)p.budget * kSelSample + n - 1) / n);
            radix_select<2>(kSelSample, kth, [&](int i) { return cval[i]; }, all, hist,
                            &sh_prefix, &sh_need);
            tau0 = sh_prefix;
        }
        // 2. Candidates in block order: each thread takes kSelPerThread
        // consecutive scores per slice, the next two slices loading while
        // this one is placed by a block scan of the per-thread counts.
        int nc = 0;
        for (int base = 0; base < n; base += kSlice) {
            float v2[kSelPerThread];
            if (base + 2 * kSlice < n) load_slice(base + 2 * kSlice, v2);
            const int i0 = base + kSelPerThread * tid;
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < kSelPerThread; ++e)
                cnt += i0 + e < n && score_key(v[e]) >= tau0;
            int total;
            const int off = block_exclusive_sum(cnt, &total, wave_sums);
            if (nc + total <= kCand) {
                int w = nc + off;
#pragma unroll
                for (int e = 0; e < kSelPerThread; ++e) {
                    if (i0 + e < n && score_key(v[e]) >= tau0) {
                        cval[cand_at(w)] = v[e];
                        cid[cand_at(w)] = i0 + e;
                        ++w;
                    }
                }
            }
            nc += total;
            __syncthreads();   // this slice's candidates are in place
#pragma unroll
            for (int e = 0; e < kSelPerThread; ++e) {
                v[e] = v1[e];
                v1[e] = v2[e];
            }
        }

        if (nc < p.budget || nc > kCand) {
            if constexpr (kDefer) {
                if (tid == 0) out[0] = kSelDeferred;
                return;
            } else {
                select_exact<false>(p, n, row, out);
                expand_row(p, pos, min(n, p.budget), out, width);
                return;
            }
        }
        select_candidates<kCand>(nc, p.budget, cval, cid, hist, &sh_prefix, &sh_need,
                                 wave_sums, kept);
    }
    expand_kept(p, pos, min(n, p.budget), kept, out, width);
}

// The selection of the fused Top-K, from the candidates indexer_scores_kernel
// kept (mode kCandidates).  One 256-thread workgroup per token: the counts of
// the token's key ranges are scanned into offsets, every range's (score,
// block id) pairs are copied in range order (so the list is in block order)
// into LDS, and the exact selection runs on them.  A row whose candidates do
// not fit their range's room, fall below the budget (the estimate was too
// high) or exceed kFusedCand is marked with kSelDeferred in its first
// output word; the full scores and the exact selection then take it
// (indexer_scores_kernel<kDeferredRows>, indexer_select_kernel<false, true>).
__global__ __launch_bounds__(256, 4) void indexer_select_cand_kernel(const IndexerSelectParams p) {
    constexpr int kCand = kFusedCand;
    constexpr int kCandPadded = kCand + kCand / 16;
    __shared__ float cval[kCandPadded];
    __shared__ int cid[kCandPadded];
    __shared__ int kept[kFusedBudgetMax];
    __shared__ int hist[256];
    __shared__ int wave_sums[4];
    __shared__ int r_off[kFusedMaxRanges + 1];
    __shared__ uint32_t sh_prefix;
    __shared__ int sh_need, sh_over;

    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    // Every range's count is written (0 past the token's eligible blocks), so
    // it is read together with the position.
    const int cnt_r = tid < p.R ? p.counts[t * p.R + tid] : 0;
    const int64_t pos = p.positions[t];
    int32_t *out = p.out + t * p.out_stride;
    const int width = kIndexBlock * p.budget + 3;
    if (pos < 0 || pos >= p.L) {
        for (int i = tid; i < width; i += 256) out[i] = -1;
        return;
    }
    const int n = (int)min<int64_t>((pos + 1) / kIndexBlock, p.C);
    if (n <= p.budget) {
        for (int e = tid; e < n; e += 256) kept[e] = e;
    } else {
        const int ranges = (n + kScoreSplit - 1) / kScoreSplit;   // <= kFusedMaxRanges
        if (tid == 0) sh_over = 0;
        __syncthreads();
        int cnt = 0;
        if (tid < ranges) {
            cnt = cnt_r;
            const int room = (int)min<int64_t>(kScoreSplit, p.C - (int64_t)tid * kScoreSplit) / 2;
            if (cnt > room) sh_over = 1;
        }
        int total;
        const int off = block_exclusive_sum(cnt, &total, wave_sums);
        if (sh_over || total < p.budget || total > kCand) {
            if (tid == 0) out[0] = kSelDeferred;
            return;
        }
        if (tid < ranges) r_off[tid] = off;
        if (tid == 0) r_off[ranges] = total;
        __syncthreads();
        // Candidate i comes from the range r with r_off[r] <= i < r_off[r + 1]
        // (a binary search); all of a thread's loads are in flight together.
        const f32x2_t *row = (const f32x2_t *)(p.scores + t * p.pair_pitch);
        constexpr int kBatch = 8;
        for (int i0 = 0; i0 < total; i0 += 256 * kBatch) {
            f32x2_t pr[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int i = i0 + 256 * k + tid;
                int lo = 0, hi = ranges;   // r_off[lo] <= i < r_off[hi]
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (r_off[mid] <= i) lo = mid;
                    else hi = mid;
                }
                if (i < total) pr[k] = row[lo * (kScoreSplit / 2) + (i - r_off[lo])];
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int i = i0 + 256 * k + tid;
                if (i < total) {
                    cval[cand_at(i)] = pr[k][0];
                    cid[cand_at(i)] = __float_as_int(pr[k][1]);
                }
            }
        }
        __syncthreads();
        select_candidates<kCand>(total, p.budget, cval, cid, hist, &sh_prefix, &sh_need,
                                 wave_sums, kept);
    }
    expand_kept(p, pos, min(n, p.budget), kept, out, width);
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerScoreParams &p, hipStream_t stream) {
    if (p.T == 0 || p.C == 0) return hipSuccess;
    const int64_t blocks = (p.T + kScoreTokens - 1) / kScoreTokens;
    const int64_t splits = (p.C + kScoreSplit - 1) / kScoreSplit;
    if (p.C % 4 == 0 && (uintptr_t)p.scores % 16 == 0 &&
        (int64_t)kScoreTokens * p.C * 4 < ((int64_t)1 << 31))
        hipLaunchKernelGGL((indexer_scores_kernel<kAllScores, true>),
                           dim3((unsigned)blocks, (unsigned)splits), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(indexer_scores_kernel<kAllScores>,
                           dim3((unsigned)blocks, (unsigned)splits), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_indexer_topk_fused(const IndexerEstimateParams &e, const IndexerScoreParams &s,
                                     const IndexerSelectParams &p, hipStream_t stream) {
    if (p.T == 0) return hipSuccess;
    if (p.budget > kFusedBudgetMax || s.R > kFusedMaxRanges || s.R < 1 || s.tau == nullptr ||
        s.deferred != nullptr || s.counts == nullptr || p.counts == nullptr)
        return hipErrorInvalidValue;
    const int64_t token_blocks = (p.T + kScoreTokens - 1) / kScoreTokens;
    hipLaunchKernelGGL(indexer_estimate_kernel, dim3((unsigned)((p.T + kEstTokens - 1) / kEstTokens)),
                       dim3(256), 0, stream, e);
    hipLaunchKernelGGL(indexer_scores_kernel<kCandidates>,
                       dim3((unsigned)token_blocks, (unsigned)s.R), dim3(256), 0, stream, s);
    hipLaunchKernelGGL(indexer_select_cand_kernel, dim3((unsigned)p.T), dim3(256), 0, stream, p);
    // Rows the estimate missed: their full scores (only workgroups holding
    // one), then the exact selection on them (the others return at once).
    IndexerScoreParams full = s;
    full.tau = nullptr;
    full.counts = nullptr;
    full.deferred = p.out;
    full.deferred_stride = p.out_stride;
    hipLaunchKernelGGL(indexer_scores_kernel<kDeferredRows>,
                       dim3((unsigned)token_blocks, (unsigned)s.R), dim3(256), 0, stream, full);
    hipLaunchKernelGGL((indexer_select_kernel<false, true>), dim3((unsigned)p.T), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_indexer_select(const IndexerSelectParams &p, hipStream_t stream) {
    if (p.T == 0) return hipSuccess;
    if (4 * (int64_t)p.budget <= kSelCandSmall) {
        hipLaunchKernelGGL((indexer_select_fast_kernel<kSelCandSmall, 4, true>),
                           dim3((unsigned)p.T), dim3(256), 0, stream, p);
        hipLaunchKernelGGL((indexer_select_kernel<false, true>), dim3((unsigned)p.T), dim3(256),
                           0, stream, p);
    } else if (4 * (int64_t)p.budget <= kSelCand)
        hipLaunchKernelGGL((indexer_select_fast_kernel<kSelCand, 4, false>), dim3((unsigned)p.T),
                           dim3(256), 0, stream, p);
    else if (p.C <= kSelectLdsBlocks)
        hipLaunchKernelGGL(indexer_select_kernel<true>, dim3((unsigned)p.T), dim3(256), 0, stream,
                           p);
    else
        hipLaunchKernelGGL(indexer_select_kernel<false>, dim3((unsigned)p.T), dim3(256), 0,
                           stream, p);
    return hipGetLastError();
}

}  // namespace qsa
