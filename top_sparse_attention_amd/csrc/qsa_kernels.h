// Internal launchers shared by the C-ABI layer and the HIP kernels.
// Not part of the public interface (that is include/qsa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Head dim the kernels are written for (the only one the method uses).
constexpr int kHeadDim = 256;
// Slots per gather tile: one 16-row MFMA block of K and V rows (16 KiB).
constexpr int kTileSlots = 16;
// Compacted lists are padded with -1 to a multiple of this.
constexpr int kListPad = 32;
// Work items (one wave each) resident per CU in the attention kernel's
// general layout.  Exactly 8 (2 per SIMD): the kernel requests enough LDS per
// item that a 9th does not fit.
// With every SIMD holding the same number of waves, the waves of a CU, and
// of the whole chip, advance through their slot-sorted lists at the same
// rate, so concurrent tokens read the same cache rows at about the same
// time and share them in L2; an uneven split (7 or 9 waves per CU) lets the
// waves drift apart and loses most of that sharing.
constexpr int kItemsPerCU = 8;
// Waves per SIMD the attention kernel's registers are budgeted for in that
// layout (up to 256 registers per wave).
constexpr int kAttendWavesPerSimd = 2;
// Tiles of gathers each attention wave keeps in flight in that layout.
constexpr int kAttendAhead = 1;
// Items per CU of the general layout when the tokens running together share
// few cache rows (see SharingParams).
constexpr int kLowShareItemsPerCU = 4;
// CUs per XCD of the MI355X (256 CUs in 8 XCDs); workgroups are dealt to the
// XCDs round robin.
constexpr int kCusPerXcd = 32;
constexpr int kXcds = 8;
// Token pairs the sharing estimate samples (at most 64: one wave adds them
// up), and the estimated sharing below which the low-sharing layout is chosen:
// kShareThreshold for lists of at least kShareLongList entries, else
// kShareThresholdShort (measured crossovers: between 4 and 8 at 1,024 and
// 2,048 entries, between 2 and 4 at 512).
constexpr int kSharePairs = 32;
constexpr float kShareThreshold = 5.0f;
constexpr float kShareThresholdShort = 3.0f;
constexpr int kShareLongList = 1024;
// The sharing at or above which BF16 items of the general layout take their
// keys through LDS (choice 2), from the estimate or from the sizes alone.
// Keys gathered as whole rows, two per load instruction like the values, touch
// 8 cache rows per instruction instead of 16; the L1 side of each CU, which
// the gathers wait on, then serves more of them.  They pass through the wave's
// LDS tile to reach the score MFMA, a round trip on each tile's path that
// costs more than it saves where most gathers miss the L2 (measured crossover
// near 8.5 on the long prefill's shape: 4% slower at 8.0, 14% faster at 10.7,
// 16-17% faster at 13 and above).
constexpr float kShareKeysLds = 9.0f;
// Splits of the decode path (decode_splits): about kDecodeUnits work units
// (one share of one item each), a wave slot each of the 4-items-per-CU
// layout; shares of at least kDecodeShareTiles tiles unless that leaves
// fewer than kDecodeMinUnits units, and never under kMinSplitTiles.  Fewer
// shares write and merge fewer partial rows (at 32 shares of a 2,048-entry
// row, the partials of 24 query heads are 38% of the K and V bytes the
// shares gather); more units keep more gathers in flight where few tokens
// run.  From kDecodeMinUnits units up, BF16 shares take the 4-items-per-CU
// layout.
constexpr int kMinSplitTiles = 4;
constexpr int kDecodeShareTiles = 8;
constexpr int kDecodeUnits = 1024;
constexpr int kDecodeMinUnits = 512;
// Entries of a selection row sorted together by the compaction pass.
constexpr int kSortThreads = 256;
constexpr int kSortItemsPerThread = 9;
constexpr int kSortChunk = kSortThreads * kSortItemsPerThread;   // 2304
// Key bits the compaction pass sorts on: the padding bit and the top 7 bits
// of the slot range (128 groups).
constexpr int kSortKeyBits = 8;
// Aligned block lists: super-ranges of about kAlignSlots cache slots (half the
// rows of one head an XCD's 4 MB L2 holds), at most kAlignMaxRanges of them
// (the sort's 128 groups); the room a row may take, kAlignRoomNum /
// kAlignRoomDen of its blocks; and the slack of the fixed start positions:
// super-range k starts near k F, F = kAlignSlackNum / kAlignSlackDen times
// the row's mean blocks per super-range (33/32: with the attention's wave
// priority the waves keep in step on their own, and 33/32 measured 2.42-2.43
// ms on the block4 long prefill against 2.43-2.44 at 17/16, 2.47-2.48 at 9/8
// and 2.58-2.59 at 5/4).
constexpr int kAlignSlots = 2048;
constexpr int kAlignMaxRanges = 1 << (kSortKeyBits - 1);
constexpr int kAlignRoomNum = 3, kAlignRoomDen = 2;
constexpr int kAlignSlackNum = 33, kAlignSlackDen = 32;
// Largest room of an aligned row (entries): the compaction builds the row in
// LDS before storing it.
constexpr int kAlignRoomMax = 4096;
// Block sizes that take the aligned lists: powers of two from kAlignMinBlock
// (2-slot blocks measured within 2%, single slots 4% slower with them) to
// kAlignMaxBlock (the attention expands list entry e of a tile row as
// slot e << log2(block) + the row's offset in the block).
constexpr int kAlignMinBlock = 4;
constexpr int kAlignMaxBlock = 64;

struct CompactParams {
    const int32_t *slot_idx;
    int64_t stride_t;
    int64_t T, W, S;
    int64_t lo, hi;      // entries in [lo, hi) are kept, stored as slot - lo
    int32_t block;       // slots per entry: entry e selects slots e*block .. e*block+block-1
                         // (S, lo, hi counted in entries of this size)
    int32_t key_bits;    // radix-sort key width: hi - lo - 1 < 2^(key_bits-1), plus one bit for padding
    // Aligned lists (align_shift >= 0; rows of at most kSortChunk entries):
    // block ids, not slots.  The entries of super-range k (entry key >>
    // align_shift, k < align_ranges <= kAlignMaxRanges, a union of the sort's
    // slot ranges) start at list position max(end of the previous ones,
    // min(k F, align_cap - entries still to place)), F = ceil(slack * row
    // entries / align_ranges); the gaps hold -1 and count[t] is the end of
    // the last.  align_cap <= row_stride.
    int32_t align_shift;
    int32_t align_ranges;
    int32_t align_cap;
    int32_t block_ids;   // aligned lists hold block ids (1) or each block's slots (0)
    int32_t *list;
    int64_t row_stride;
    int32_t *count;
    int32_t *n_bad;
    // Workspace words [2], written by workgroup 0: the number of cache slots
    // the lists index, (hi - lo) * block (every list entry is below it), and
    // a cleared flag that an attention over a smaller cache view sets.
    int32_t *extent;
};

// Element type of the K/V cache: BF16, or FP8 E4M3 codes with one scale per
// tensor (the softmax scale absorbs k_scale; v_scale multiplies the output).
enum class KvType { kBf16, kFp8 };

struct AttendParams {
    const uint16_t *q;
    int64_t q_st, q_sh;
    const void *k;       // [S, Hkv, 256] of the KV type; strides in elements
    int64_t k_ss, k_sh;
    const void *v;
    int64_t v_ss, v_sh;
    float v_scale;       // FP8 only
    const int32_t *list;
    int64_t list_stride;
    const int32_t *count;
    uint16_t *out;
    int64_t o_st, o_sh;
    int32_t Hkv;
    int32_t G;           // query heads per KV head
    int32_t HB;          // 16-head blocks per KV head: ceil(G / 16)
    float scale_log2e;   // scale * log2(e)
    // Split mode only: each item's tiles are dealt to `splits` workgroups, and
    // workgroup s writes partial (O, m, l) to part (part_base + s).
    int32_t splits;
    int64_t part_base;
    int64_t T;
    int32_t Hq;
    float *part_o;       // [n_parts][T][Hq][256], O not yet divided by l
    float *part_ml;      // [n_parts][T][Hq][2]: running max (log2 units) and sum
    // Gated launch (non-null choice): the kernel does its work only if
    // *choice == choice_value; the sharing estimate writes the word (0, 1 or
    // 2) before the gated launches, so exactly one of them works.
    const int32_t *choice;
    int32_t choice_value;
    // Ungated BF16 launch of the general layout: keys_lds = 1 takes its
    // keys-through-LDS form (see SharingParams), which computes the same bits.
    int32_t keys_lds;
    // Work units of the launch (items, times splits in split mode); set by
    // the launcher, which sizes the grid.
    int64_t units;
    // Unsplit items over a compacted list with -1 gaps (the aligned block
    // lists; masked = 1, BF16, S_rows = S): entries are masked per tile row.
    // Each entry is a block of 2^block_shift slots; count[t] counts entries.
    int32_t masked;
    int32_t block_shift;
    // Split mode over raw selection rows (raw_rows = 1): each share
    // reads slot_idx row t itself (W_raw entries, -1 and invalid entries
    // included; valid means in [0, S_rows)) instead of a compacted list, and
    // the share with g = 0 and head block 0 writes its count of invalid
    // entries to bad_part[split * T + t].
    // (The mode is the flag, not raw's nullness: a zero-width row set has no
    // data pointer, and its shares read nothing.)
    int32_t raw_rows;
    const int32_t *raw;
    int64_t raw_stride;
    int32_t W_raw;
    int64_t S_rows;      // slots of the k/v views
    int32_t *bad_part;
    // Compacted lists: the workspace's extent words (see CompactParams).  An
    // item whose lists index more slots than S_rows reads nothing, writes a
    // zero row (or an empty share) and sets extent[1].  Unused for raw rows.
    int32_t *extent;
};

// Sharing estimate.  Items run kItemsPerCU to a CU and walk their slot lists
// in ascending slot ranges at about the same rate, so a cache row one item
// reads is read at about the same time by the other items on its XCD that
// read it, and they share it in L2.  The expected number of such readers is
//   lambda = (concurrent items of one KV head per XCD) x |L_a & L_b| / |L_b|
// for tokens a, b that run together.  The estimate takes `pairs` token
// pairs (pair_a[i], pair_b[i]), counts each pair's common slots, and writes
// choice = 1 (take the kLowShareItemsPerCU layout) if
// lambda_scale * sum|L_a & L_b| < threshold * sum|L_b|; else choice = 2 (the
// general layout with keys through LDS) if lds_threshold > 0 and
// lambda_scale * sum|L_a & L_b| >= lds_threshold * sum|L_b|; else 0.
struct SharingParams {
    const int32_t *list;
    int64_t row_stride;
    const int32_t *count;
    int32_t pairs;
    int32_t pair_a[kSharePairs], pair_b[kSharePairs];   // token rows, a != b
    float lambda_scale;   // concurrent items of one KV head per XCD
    float threshold;
    float lds_threshold;  // 0: no keys-through-LDS form (FP8 caches)
    float *est;           // [pairs][2]: common slots (scaled), |L_b|
    int32_t *choice;
};

struct MergeParams {
    const float *part_o;
    const float *part_ml;
    int64_t n_parts, T;
    int32_t Hq;
    uint16_t *out;
    int64_t o_st, o_sh;
    // Non-null after raw-row shares: n_bad[t] = sum over parts of bad_part[s * T + t].
    const int32_t *bad_part;
    int32_t *n_bad;
    // Non-null: workgroup 0 writes 0 here (the workspace's extent flag, which
    // no compaction of a decode step clears).
    int32_t *clear_flag;
};

struct GatherParams {
    const void *k;
    int64_t k_ss, k_sh;
    const void *v;
    int64_t v_ss, v_sh;
    const int32_t *list;
    int64_t list_stride;
    const int32_t *count;
    uint32_t *sink;
    int32_t Hkv;
    int64_t S_rows;              // slots of the k/v views
    const int32_t *extent;       // the workspace's extent word (see CompactParams)
};

hipError_t launch_compact(const CompactParams &p, hipStream_t stream);
// With a non-null `share`, the sharing estimate runs first and picks the
// layout (general-layout kernels only; others ignore it).
hipError_t launch_attend(const AttendParams &p, KvType kv, int64_t T, hipStream_t stream,
                         const SharingParams *share = nullptr);
hipError_t launch_attend_partial(const AttendParams &p, KvType kv, int64_t T,
                                 hipStream_t stream);
hipError_t launch_merge(const MergeParams &p, hipStream_t stream);
hipError_t launch_gather_only(const GatherParams &p, KvType kv, int64_t T, hipStream_t stream);

}  // namespace qsa
