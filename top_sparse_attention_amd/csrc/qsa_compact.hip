// Index validation and compaction for QSA sparse main-attention prefill
// (gfx950): the pass that turns each token's selection row into the list of
// slots the attention gathers.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include <hipcub/block/block_load.hpp>
#include <hipcub/block/block_radix_sort.hpp>

#include "qsa_device.h"
#include "qsa_kernels.h"

namespace qsa {
namespace {

// One workgroup per token row.  Entries in [lo, hi) are kept and stored as
// slot - lo (a cache shard's local numbering; lo = 0, hi = S keeps them
// all); entries that are neither -1 nor in [0, S) are counted as invalid.
// With block > 1 an entry names a micro-block of `block` consecutive slots
// (S, lo, hi then count blocks) and expands to those slots in order.
// The row is processed in chunks of
// kSortChunk entries; each chunk's valid slots are radix-sorted on the top
// kSortKeyBits bits of a key_bits-wide key (invalid entries carry the key
// 2^(key_bits-1), so they sort last), i.e. grouped into at most 128 ascending
// slot ranges, stable inside a range, and appended to the compacted list.
// Two radix passes; a full sort would cost more and buys no locality.
// Aligned lists (align_shift >= 0, one run per row) place each super-range of
// about kAlignSlots slots near a fixed position of the row instead, the gaps
// holding -1: the tokens running at one time, whose lists have different
// counts per range, then reach each part of the cache after about the same
// number of tiles (their gathers share the L2), at about 25% more tiles.
template <bool kAligned>
__global__ __launch_bounds__(kSortThreads) void compact_kernel(const CompactParams p) {
    using Load = hipcub::BlockLoad<int32_t, kSortThreads, kSortItemsPerThread,
                                   hipcub::BLOCK_LOAD_TRANSPOSE>;
    using Sort = hipcub::BlockRadixSort<uint32_t, kSortThreads, kSortItemsPerThread>;
    __shared__ union {
        typename Load::TempStorage load;
        typename Sort::TempStorage sort;
    } tmp;
    __shared__ int chunk_counts;   // valid entries | invalid entries << 16
    // Aligned lists: per super-range its entry count, first rank, the start
    // of the gap before it and its start (slot positions); the row's end.
    __shared__ int sr_cnt[kAlignMaxRanges], sr_first[kAlignMaxRanges];
    __shared__ int sr_gap[kAlignMaxRanges], sr_start[kAlignMaxRanges];
    __shared__ int sh_end;
    // Aligned lists: the row is built here (gaps -1) and stored in one pass.
    __shared__ int row_stage[kAligned ? kAlignRoomMax : 1];

    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    if (t == 0 && tid == 0) {
        // Every list entry is below this; an attention over a cache view with
        // fewer slots refuses the lists (and sets the flag cleared here).
        p.extent[0] = (int32_t)((p.hi - p.lo) * p.block);
        p.extent[1] = 0;
    }
    const int32_t *src = p.slot_idx + t * p.stride_t;
    int32_t *dst = p.list + t * p.row_stride;
    const uint32_t pad_key = 1u << (p.key_bits - 1);
    const bool aligned = kAligned && p.W <= kSortChunk && p.align_cap <= kAlignRoomMax;
    int n = 0, bad = 0, aligned_end = 0;
    for (int64_t base = 0; base < p.W; base += kSortChunk) {
        if (tid == 0) chunk_counts = 0;
        // Coalesced loads, handed to the sort in blocked order (thread t holds
        // entries 9t .. 9t + 8 of the run), so the sort is stable in the
        // row's order.
        int32_t e[kSortItemsPerThread];
        Load(tmp.load).Load(src + base, e, (int)min<int64_t>(kSortChunk, p.W - base), -1);
        __syncthreads();   // the load's staging area is reused by the sort
        uint32_t key[kSortItemsPerThread];
        int my_valid = 0, my_bad = 0;
#pragma unroll
        for (int u = 0; u < kSortItemsPerThread; ++u) {
            const bool in_cache = e[u] >= 0 && (int64_t)e[u] < p.S;
            const bool keep = in_cache && (int64_t)e[u] >= p.lo && (int64_t)e[u] < p.hi;
            my_valid += keep;
            my_bad += !in_cache && e[u] != -1;
            key[u] = keep ? (uint32_t)((int64_t)e[u] - p.lo) : pad_key;
        }
        // Both counts (each < 2^16 per run) in one word, summed per wave.
        int packed = my_valid | (my_bad << 16);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) packed += __shfl_xor(packed, off);
        if ((tid & 63) == 0) atomicAdd(&chunk_counts, packed);
        // Sorted keys come back striped: thread t holds ranks t, t + 256, ...,
        // so the stores below are coalesced.
        Sort(tmp.sort).SortBlockedToStriped(key, max(p.key_bits - kSortKeyBits, 0), p.key_bits);
        __syncthreads();   // the counts above are complete
        const int nv = chunk_counts & 0xffff;
        const int nb = chunk_counts >> 16;
        if (aligned) {
            // One run holds the row.  Entries per super-range, then (one
            // thread, at most kAlignMaxRanges steps) where each starts.
            for (int i = tid; i < kAlignMaxRanges; i += kSortThreads) sr_cnt[i] = 0;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kSortItemsPerThread; ++u) {
                const int pos = tid + kSortThreads * u;
                if (pos < nv) atomicAdd(&sr_cnt[min((int)(key[u] >> p.align_shift), p.align_ranges - 1)], 1);
            }
            __syncthreads();
            if (tid == 0) {
                const int slots = nv * p.block, R = p.align_ranges;
                const int F = (5 * slots + 4 * R - 1) / (4 * R);   // 1.25 x the mean, rounded up
                int end = 0, first = 0, rem = slots;
                for (int k = 0; k < R; ++k) {
                    const int cs = sr_cnt[k] * p.block;
                    // end + rem <= align_cap holds before and after each step.
                    const int start = cs > 0 ? max(end, min(k * F, p.align_cap - rem)) : end;
                    sr_gap[k] = end;
                    sr_start[k] = start;
                    sr_first[k] = first;
                    end = start + cs;
                    first += sr_cnt[k];
                    rem -= cs;
                }
                sh_end = end;
            }
            __syncthreads();
            // The row up to its padded end: -1 everywhere, then the entries at
            // their places, then one coalesced store of the whole row.
            const int row_end = (sh_end + kListPad - 1) / kListPad * kListPad;   // <= align_cap
            for (int i = tid; i < row_end; i += kSortThreads) row_stage[i] = -1;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kSortItemsPerThread; ++u) {
                const int pos = tid + kSortThreads * u;
                if (pos < nv) {
                    const int k = min((int)(key[u] >> p.align_shift), p.align_ranges - 1);
                    const int at = sr_start[k] + (pos - sr_first[k]) * p.block;
                    for (int i = 0; i < p.block; ++i)
                        if ((unsigned)(at + i) < (unsigned)row_end)
                            row_stage[at + i] = (int32_t)key[u] * p.block + i;
                }
            }
            __syncthreads();
            for (int i = tid; i < row_end; i += kSortThreads) dst[i] = row_stage[i];
            aligned_end = sh_end;
        } else if (p.block == 1) {
#pragma unroll
            for (int u = 0; u < kSortItemsPerThread; ++u) {
                const int pos = tid + kSortThreads * u;
                if (pos < nv) dst[n + pos] = (int32_t)key[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < kSortItemsPerThread; ++u) {
                const int pos = tid + kSortThreads * u;
                if (pos < nv)
                    for (int i = 0; i < p.block; ++i)
                        dst[(int64_t)(n + pos) * p.block + i] = (int32_t)key[u] * p.block + i;
            }
        }
        n += nv;
        bad += nb;
        __syncthreads();   // the counts are reset by the next run
    }
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
