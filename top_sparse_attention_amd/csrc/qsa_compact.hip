// Index validation and compaction for QSA sparse main-attention prefill
// (gfx950): the pass that turns each token's selection row into the list of
// slots the attention gathers.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include "qsa_device.h"
#include "qsa_kernels.h"

namespace qsa {
namespace {

// One workgroup per token row.  Entries in [lo, hi) are kept and stored as
// slot - lo (a cache shard's local numbering; lo = 0, hi = S keeps them
// all); entries that are neither -1 nor in [0, S) are counted as invalid.
// With block > 1 an entry names a micro-block of `block` consecutive slots
// (S, lo, hi then count blocks) and expands to those slots in order.
// The row is processed in runs of kSortChunk entries; each run's kept
// entries are grouped by their top bits, group = key >> max(key_bits - 8, 0)
// (at most kGroups ascending slot ranges), stably (input order inside a
// group), and appended to the compacted list.  A full sort would cost more
// and buys no locality.
//
// The grouping is a counting sort written for 64-lane waves: wave w takes the
// run's entries [w kWaveRun, (w + 1) kWaveRun) as 9 slices of 64 consecutive
// entries (one per lane, coalesced loads).  Per slice the lanes holding the
// same group find each other with one ballot per group bit, rank themselves
// by the lanes below them, and the lowest of them adds the slice's count to
// the wave's running count of that group (LDS, private to the wave, so no
// barrier inside the loop).  One wave then scans the 4 x kGroups counts into
// output offsets, and every entry lands at offset + rank in an LDS copy of
// the run, which is stored with coalesced writes.
//
// Aligned lists (align_shift >= 0, one run per row; micro-block selections)
// hold block ids, not slots: each super-range of about kAlignSlots slots
// starts near a fixed position of the row, the gaps holding -1, so the tokens
// running at one time, whose lists have different counts per range, reach
// each part of the cache after about the same number of tiles (their gathers
// share the L2).  The attention expands each block into its slots.
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kWaveRun = kSortChunk / kSortWaves;        // 576 entries per wave
constexpr int kSlices = kWaveRun / 64;                   // 9
constexpr int kGroups = 1 << (kSortKeyBits - 1);         // 128
constexpr int kGroupBits = kSortKeyBits - 1;             // bits of a kept entry's group
static_assert(kSortChunk % kSortThreads == 0 && kWaveRun % 64 == 0, "run layout");
static_assert(kGroups == 2 * 64, "the offset scan gives each lane two groups");

template <bool kAligned>
__global__ __launch_bounds__(kSortThreads) void compact_kernel(const CompactParams p) {
    // Per wave and group: the running count while ranking, then the run's
    // output offset of that wave's entries of that group.
    __shared__ int wave_cnt[kSortWaves][kGroups];
    __shared__ int group_first[kGroups];        // sorted position of each group's first entry
    __shared__ int wave_valid[kSortWaves], wave_bad[kSortWaves];
    // The run in its output order (plain lists), or the whole aligned row.
    __shared__ int stage[kAligned ? kAlignRoomMax : kSortChunk];
    // Aligned lists: per super-range its entry count, first rank and start
    // (list position, in blocks); the row's end.
    __shared__ int sr_cnt[kAlignMaxRanges], sr_first[kAlignMaxRanges], sr_start[kAlignMaxRanges];
    __shared__ int sh_end;

    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    if (t == 0 && tid == 0) {
        // Every list entry is below this; an attention over a cache view with
        // fewer slots refuses the lists (and sets the flag cleared here).
        p.extent[0] = (int32_t)((p.hi - p.lo) * p.block);
        p.extent[1] = 0;
    }
    const int32_t *src = p.slot_idx + t * p.stride_t;
    int32_t *dst = p.list + t * p.row_stride;
    const int gshift = max(p.key_bits - kSortKeyBits, 0);
    const bool aligned = kAligned && p.W <= kSortChunk && p.align_cap <= kAlignRoomMax;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int n = 0, bad = 0, aligned_end = 0;
    for (int64_t base = 0; base < p.W; base += kSortChunk) {
        // The wave's entries of this run, all loads in flight together.
        const int64_t wbase = base + (int64_t)kWaveRun * wave + lane;
        int32_t e[kSlices];
#pragma unroll
        for (int u = 0; u < kSlices; ++u) {
            const int64_t i = wbase + 64 * u;
            e[u] = i < p.W ? src[i] : -1;
        }
        for (int i = lane; i < kGroups; i += 64) wave_cnt[wave][i] = 0;
        // e[u] becomes the kept entry's key (slot - lo), or -1 if dropped;
        // rank[u] its rank among the wave's entries of its group.
        int rank[kSlices];
        int my_valid = 0, my_bad = 0;
#pragma unroll
        for (int u = 0; u < kSlices; ++u) {
            // 32-bit tests (the host keeps S below 2^31 and 0 <= lo <= hi <= S).
            const int x = e[u];
            const bool in_cache = (uint32_t)x < (uint32_t)p.S;
            const bool keep = (uint32_t)(x - (int)p.lo) < (uint32_t)(p.hi - p.lo);
            my_valid += keep;
            my_bad += !in_cache && x != -1;
            const int key = x - (int)p.lo;
            e[u] = keep ? key : -1;
            const int g = key >> gshift;
            // Lanes of this slice holding group g (kept entries only: the
            // others are out of the first ballot, so 7 group bits suffice).
            uint64_t same = __ballot(keep);
#pragma unroll
            for (int b = 0; b < kGroupBits; ++b) {
                const int bit = __builtin_amdgcn_sbfe(g, b, 1);   // 0 or -1
                same &= ~(__ballot(bit) ^ (uint64_t)(int64_t)bit);
            }
            // Previous slices' count of g in this wave, then this slice's.
            const int before = keep ? wave_cnt[wave][g & (kGroups - 1)] : 0;
            rank[u] = before + __popcll(same & below);
            if (keep && (same & below) == 0) wave_cnt[wave][g] = before + __popcll(same);
            // One slice at a time: interleaving them would only hold more
            // masks in registers, since each waits for the previous one's count.
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            my_valid += __shfl_xor(my_valid, off);
            my_bad += __shfl_xor(my_bad, off);
        }
        if (lane == 0) {
            wave_valid[wave] = my_valid;
            wave_bad[wave] = my_bad;
        }
        __syncthreads();   // every wave's counts are in place
        if (wave == 0) {
            // Lane l owns groups 2l and 2l + 1: their totals over the waves,
            // an exclusive scan over the groups, then each wave's offset.
            int c0[kSortWaves], c1[kSortWaves], t0 = 0, t1 = 0;
#pragma unroll
            for (int w = 0; w < kSortWaves; ++w) {
                c0[w] = wave_cnt[w][2 * lane];
                c1[w] = wave_cnt[w][2 * lane + 1];
                t0 += c0[w];
                t1 += c1[w];
            }
            int incl = t0 + t1;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(incl, off);
                if (lane >= off) incl += v;
            }
            int at0 = incl - t0 - t1, at1 = at0 + t0;
            group_first[2 * lane] = at0;
            group_first[2 * lane + 1] = at1;
#pragma unroll
            for (int w = 0; w < kSortWaves; ++w) {
                wave_cnt[w][2 * lane] = at0;
                wave_cnt[w][2 * lane + 1] = at1;
                at0 += c0[w];
                at1 += c1[w];
            }
        }
        __syncthreads();   // offsets are in place
        const int nv = wave_valid[0] + wave_valid[1] + wave_valid[2] + wave_valid[3];
        const int nb = wave_bad[0] + wave_bad[1] + wave_bad[2] + wave_bad[3];
        if (aligned) {
            // One run holds the row.  Entries per super-range, then (one
            // thread, at most kAlignMaxRanges steps) where each starts.
            const int per_sr = p.align_shift - gshift;   // groups per super-range: 2^per_sr
            for (int k = tid; k < p.align_ranges; k += kSortThreads) {
                const int g0 = min(k << per_sr, kGroups), g1 = min((k + 1) << per_sr, kGroups);
                const int first = g0 < kGroups ? group_first[g0] : nv;
                const int last = g1 < kGroups ? group_first[g1] : nv;
                sr_first[k] = first;
                sr_cnt[k] = k == p.align_ranges - 1 ? nv - first : last - first;
            }
            __syncthreads();
            // List entries per kept block: 1 (block ids) or the block's slots.
            const int unit = p.block_ids ? 1 : p.block;
            if (tid == 0) {
                const int R = p.align_ranges;
                // F = the mean entries per super-range times the slack, rounded up.
                const int F = (kAlignSlackNum * nv * unit + kAlignSlackDen * R - 1) /
                              (kAlignSlackDen * R);
                int end = 0, rem = nv * unit;
                for (int k = 0; k < R; ++k) {
                    const int cs = sr_cnt[k] * unit;
                    // end + rem <= align_cap holds before and after each step.
                    const int start = cs > 0 ? max(end, min(k * F, p.align_cap - rem)) : end;
                    sr_start[k] = start;
                    end = start + cs;
                    rem -= cs;
                }
                sh_end = end;
            }
            __syncthreads();
            // The row up to its padded end: -1 everywhere, then the entries at
            // their places, then one coalesced store of the whole row.
            const int row_end = (sh_end + kListPad - 1) / kListPad * kListPad;   // <= align_cap
            for (int i = tid; i < row_end; i += kSortThreads) stage[i] = -1;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kSlices; ++u) {
                if (e[u] >= 0) {
                    const int g = e[u] >> gshift;
                    const int pos = wave_cnt[wave][g] + rank[u];
                    const int k = min(g >> per_sr, p.align_ranges - 1);
                    const int at = sr_start[k] + (pos - sr_first[k]) * unit;
                    for (int i = 0; i < unit; ++i)
                        if ((unsigned)(at + i) < (unsigned)row_end)
                            stage[at + i] = p.block_ids ? e[u] : e[u] * p.block + i;
                }
            }
            __syncthreads();
            for (int i = tid; i < row_end; i += kSortThreads) dst[i] = stage[i];
            aligned_end = sh_end;
        } else {
#pragma unroll
            for (int u = 0; u < kSlices; ++u)
                if (e[u] >= 0) stage[wave_cnt[wave][e[u] >> gshift] + rank[u]] = e[u];
            __syncthreads();
            if (p.block == 1) {
                for (int i = tid; i < nv; i += kSortThreads) dst[n + i] = stage[i];
            } else {
                for (int i = tid; i < nv; i += kSortThreads)
                    for (int b = 0; b < p.block; ++b)
                        dst[(int64_t)(n + i) * p.block + b] = stage[i] * p.block + b;
            }
        }
        n += nv;
        bad += nb;
        __syncthreads();   // the run's LDS is reused by the next run
    }
    // count[t]: list entries (blocks) of an aligned row, else slots.
    const int slots = aligned ? aligned_end : n * p.block;
    const int padded = (slots + kListPad - 1) / kListPad * kListPad;
    for (int i = slots + tid; i < padded; i += kSortThreads) dst[i] = -1;
    if (tid == 0) {
        p.count[t] = slots;
        p.n_bad[t] = bad;
    }
}

}  // namespace

hipError_t launch_compact(const CompactParams &p, hipStream_t stream) {
    if (p.T == 0) return hipSuccess;
    if (p.align_shift >= 0) {
        if (p.W > kSortChunk || p.align_cap > kAlignRoomMax) return hipErrorInvalidValue;
        hipLaunchKernelGGL(compact_kernel<true>, dim3((unsigned)p.T), dim3(kSortThreads), 0,
                           stream, p);
    } else {
        hipLaunchKernelGGL(compact_kernel<false>, dim3((unsigned)p.T), dim3(kSortThreads), 0,
                           stream, p);
    }
    return hipGetLastError();
}


}  // namespace qsa
