// Attention kernels for QSA sparse main-attention prefill on gfx950 (MI355X, CDNA4).
//
// The operation is the one on the page "Qwen4-Exp QSA comes to Huawei's
// Ascend: inside SGLang's opt-in CANN prefill PR", section "What the pull
// request actually adds": softmax(scale * Q K^T) V, where each query token
// sees only the physical cache slots its indexer selected.  Unlike the
// page's adapter this code packs nothing: it gathers the selected K and V rows
// in place, takes any query/KV head ratio without padding it to a power of
// two, and needs no host synchronisation.
//
// The prefill path is two passes:
//  1. compact_kernel: per token row, keep the entries in [0, S) (counting
//     the others as invalid), group them into ascending slot ranges (a
//     partial radix sort), and pad the list with -1 to a multiple of
//     kListPad.  The order does not change the result (the softmax sum is
//     order-free) but makes each wave's consecutive gathers land in few
//     large pages of the cache, and lets the tokens running at one time
//     read the same rows at about the same time.
//  2. attend_kernel: one work item = (token t, KV head g, block of up to 16
//     query heads of that group) = one wave, 8 items resident per CU (4
//     where sharing_kernel estimates that the running tokens share few
//     cache rows; 12 for FP8 caches with at most 8 heads per KV head; see
//     AttendLayout).  The wave walks its item's 16-slot tiles in
//     list order.  Per tile it loads the K rows straight into the registers
//     of the score MFMA's A operand and the V rows (whole rows) into
//     registers that it then writes to its LDS tile, both one tile ahead of
//     use; computes the 16x16 score tile with bf16 MFMA (K rows x query
//     heads, the query rows read from LDS), runs an online softmax in FP32
//     and accumulates P.V with bf16 MFMA fed by LDS transpose loads, then
//     writes the row in BF16.  Where the running tokens share many rows
//     (BF16), the keys come as whole rows through the LDS tile instead
//     (kKeysLds).  Its split form writes FP32 (O, m, l) partials of a share
//     of the tiles instead, which merge_kernel (or merge_rows_kernel)
//     combines.
// This file holds the attention kernels, their merge, the sharing estimate
// and gather_only_kernel (the attention's loads alone, a measurement aid);
// qsa_compact.hip holds the compaction pass and qsa_indexer.hip the QSA
// indexer that produces the selection (index scores with bf16 MFMA and the
// Top-K selection kernels).

// MFMA orientation: scores are computed transposed, S^T = K_tile . Q^T, so
// that one lane owns one query head (column) of the MFMA output: the row
// maximum needs only two cross-lane steps and the O rescale is one scalar per
// lane.  The output O^T = V^T . P^T uses the same lane-to-head map, and the
// 16x16 score tile in MFMA output layout is directly the P^T operand of the
// 16x16x16 MFMA.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <stdint.h>

#include "qsa_device.h"
#include "qsa_kernels.h"

namespace qsa {
namespace {

constexpr int kRowBytes = kHeadDim * 2;             // one BF16 row: 512 B
constexpr int kChunksPerRow = kRowBytes / 16;       // 32 sixteen-byte chunks

// LDS row pitch of the query rows (528 B = 33 chunks: the 8 rows read by
// one phase of a 16-byte read start in 8 different 16-byte bank groups).
// Rows are padded rather than swizzled, so every LDS access of the tile loop
// is one per-lane base address plus an immediate offset.
constexpr int kQPitch = kRowBytes + 16;

// How one tile of a cache with this element type is gathered.
//  K: 16 rows in MFMA A-operand layout; every lane loads 16 bytes per load
//     instruction from its row (see gather_k for which bytes).
//  V: whole rows, each row split into 16-byte chunks, one per lane,
//     kRowsPerLoad rows per load instruction.
template <KvType KV>
struct KvGather {
    static constexpr int kElemBytes = KV == KvType::kFp8 ? 1 : 2;
    static constexpr int kRowBytesHbm = kHeadDim * kElemBytes;  // 512 or 256
    static constexpr int kKLoads = kRowBytesHbm / 64;             // 8 or 4
    static constexpr int kLanesPerRow = kRowBytesHbm / 16;        // 32 or 16
    static constexpr int kRowsPerLoad = 64 / kLanesPerRow;        // 2 or 4
    static constexpr int kVLoads = kTileSlots / kRowsPerLoad;     // 8 or 4
};
constexpr int kHeadBlock = 16;                      // query heads per MFMA column block
constexpr int kDimBlocks = kHeadDim / 16;           // 16 output blocks of 16 dims
constexpr int kKSteps = kHeadDim / 32;              // 8 k-steps of the score MFMA
// A new running maximum is adopted only when it exceeds the current one by
// more than this (log2 units); otherwise probabilities may reach 2^8, which
// FP32 sums and BF16 probabilities hold exactly as well.  This skips most
// rescales of the O accumulators.
constexpr float kRescaleSlack = 8.0f;

// LDS layout and residency of one attention item (one wave): its V tile and
// kQRows query rows.
//  kQRows = 16 (any head ratio): V rows of 544 B (136 banks: the 4 rows one
//    16-lane group reads with a transpose load fall in 4 different 32-byte
//    bank windows; 8 lanes writing consecutive chunks of a row hit 8 different
//    16-byte bank groups).  The item requests a block sized so that exactly
//    kItems items fit in the 160 KiB of a CU: kItemsPerCU, or
//    kLowShareItemsPerCU where the running tokens share few cache rows.
//  kQRows = 8 (FP8 caches with at most 8 query heads per KV head): V rows of
//    528 B; the 12.4 KiB item lets 12 items (3 per SIMD) fit a CU.  FP8
//    tiles are short and their waves wait on load latency, which the extra
//    items hide (BF16 measured slower this way).  MFMA columns 8..15 then
//    repeat heads 0..7 and are not written out.
template <int kQRows, int kItemsGeneral = kItemsPerCU>
struct AttendLayout {
    static constexpr int kVPitch = kQRows == 16 ? kRowBytes + 32 : kRowBytes + 16;
    static constexpr int kTileBytes = kTileSlots * kVPitch;
    static constexpr int kQBytes = kQRows * kQPitch;
    static constexpr int kUsed = kTileBytes + kQBytes;
    static constexpr int kItems = kQRows == 16 ? kItemsGeneral : 12;
    static constexpr int kLds = kQRows == 16 ? 160 * 1024 / kItems - 1024 : kUsed;
    static constexpr int kWavesPerSimd = kQRows == 16 ? (kItems >= 8 ? kAttendWavesPerSimd : 1) : 3;
    static constexpr int kAhead = kQRows == 16 ? kAttendAhead : 1;   // tiles in flight per wave
    // Persistent workgroups (see attend_kernel): the 4-per-CU layout.
    static constexpr bool kPersistent = kItems == kLowShareItemsPerCU;
    static constexpr int kQChunksPerLane = kQRows * kChunksPerRow / 64;
    static_assert(kUsed <= kLds, "item LDS");
    static_assert(kItems * kLds <= 160 * 1024, "LDS budget of a gfx950 CU");
    // with the 1,280-byte LDS allocation granule
    static_assert((kItems + 1) * ((kLds + 1279) / 1280 * 1280) > 160 * 1024,
                  "one more item must not fit");
};

// ---------------------------------------------------------------- gathers

// Start of the cache row of `slot` (a valid slot: see stand_in).
// The slot is at least 0 and the slot stride (bytes) under 2^32 (the host
// checks it), so one unsigned 32 x 32 -> 64-bit multiply-add forms it.
__device__ __forceinline__ const char *row_ptr(const char *base, uint32_t ss, int slot) {
    return base + (uint64_t)(uint32_t)slot * ss;
}

// K rows go straight from memory into the A operand of the score MFMA.  The
// dims of the head are grouped into the 8 k-steps so that one 16-byte load
// of FP8 codes feeds two k-steps: k-step ks = 2u + b of lane group j takes
// dims 64 u + 16 j + 8 b .. +8.  BF16 keys use the same grouping (so both
// cache types give the same sums), each lane loading those 8 dims (16
// bytes) per k-step: the loads of k-steps 2u and 2u + 1 together read 128
// contiguous bytes of each of the 16 rows.  FP8 keys: load u reads dims
// 64 u + 16 j .. +16, converted just before use.  The query operand of each
// k-step is read with the same map (q_chunk).  `slot` is the slot of tile
// row (lane & 15), from stand_in.
template <KvType KV>
__device__ __forceinline__ void gather_k1(u32x4_t &r, int q, int slot, const char *kb,
                                          uint32_t k_ss, int lane) {
    const int j = lane >> 4;
    const char *row = row_ptr(kb, k_ss, slot);
    if constexpr (KV == KvType::kBf16)
        r = ldg16<u32x4_t>(row + 128 * (q >> 1) + 32 * j + 16 * (q & 1));
    else
        r = ldg16<u32x4_t>(row + 64 * q + 16 * j);
}

template <KvType KV>
__device__ __forceinline__ void gather_k(u32x4_t (&rk)[KvGather<KV>::kKLoads], int slot,
                                         const char *kb, uint32_t k_ss, int lane) {
#pragma unroll
    for (int q = 0; q < KvGather<KV>::kKLoads; ++q) gather_k1<KV>(rk[q], q, slot, kb, k_ss, lane);
}

// The 16-byte chunk (8 dims) of a query row that pairs with k-step ks of
// lane group j, following gather_k.
__device__ __forceinline__ constexpr int q_chunk(int ks, int j) {
    return 8 * (ks >> 1) + 2 * j + (ks & 1);
}

// 8 FP8 E4M3 codes (two dwords) -> 8 BF16 values (exact: every E4M3 value is
// a BF16 value).  v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two codes
// per instruction; it matches the two-step conversion through FP32 on all
// 256 codes in every byte position (checked on the GPU).
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The maximum of x over the four lane groups of a column (lanes c, c + 16,
// c + 32, c + 48), with the row-swap instructions of gfx950 (vector ALU, no
// trip through the LDS as a lane shuffle takes).  Swapping a value with
// itself leaves every lane holding its own value and its partner's, in an
// order that depends on the lane; fmaxf takes both.
__device__ __forceinline__ float max_over_lane_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// A operand of k-step ks from the K registers.
template <KvType KV>
__device__ __forceinline__ bf16x8_t k_operand(const u32x4_t (&rk)[KvGather<KV>::kKLoads], int ks) {
    if constexpr (KV == KvType::kBf16) {
        return __builtin_bit_cast(bf16x8_t, rk[ks]);
    } else {
        const u32x4_t w = rk[ks >> 1];
        return (ks & 1) ? fp8x8_to_bf16(w[2], w[3]) : fp8x8_to_bf16(w[0], w[1]);
    }
}

// V rows are read whole: load q covers kRowsPerLoad consecutive tile rows,
// each read by kLanesPerRow consecutive lanes, 16 bytes per lane, so every
// row is one fully coalesced read.  The slot of each row is broadcast from
// the lane that holds it.  Each load is issued right after its own address
// work and nothing is moved across it: the loads of a wave reach the memory
// system spread out rather than as one burst, which measured markedly faster
// (a burst of whole-row loads from every wave delays the other waves'
// requests and lets the waves of the chip fall out of step).
template <KvType KV, bool kScalarAddr>
__device__ __forceinline__ void gather_v(u32x4_t (&rv)[KvGather<KV>::kVLoads], int slot,
                                         const char *vb, uint32_t v_ss, int lane) {
    using G = KvGather<KV>;
    const int byte_in_row = (lane % G::kLanesPerRow) * 16;
    const int sub = lane / G::kLanesPerRow;   // which row of the load this lane reads
#pragma unroll
    for (int q = 0; q < G::kVLoads; ++q) {
        // The slots of the load's rows are wave-uniform (read from the lanes
        // that hold them).  kScalarAddr: each row's address is formed in
        // scalar registers (the empty asm keeps it there) and each lane picks
        // the one of its row.  Otherwise each lane picks its row's slot and
        // forms the address with vector instructions.  Which is faster
        // depends on the layout (see the attention kernel).
        uint64_t row;
        if constexpr (kScalarAddr) {
            uint64_t addr[G::kRowsPerLoad];
#pragma unroll
            for (int r = 0; r < G::kRowsPerLoad; ++r) {
                addr[r] = (uint64_t)row_ptr(
                    vb, v_ss, __builtin_amdgcn_readlane(slot, G::kRowsPerLoad * q + r));
                asm volatile("" : "+s"(addr[r]));
            }
            row = addr[0];
#pragma unroll
            for (int r = 1; r < G::kRowsPerLoad; ++r) row = sub == r ? addr[r] : row;
        } else {
            int s = __builtin_amdgcn_readlane(slot, G::kRowsPerLoad * q);
#pragma unroll
            for (int r = 1; r < G::kRowsPerLoad; ++r) {
                const int sr = __builtin_amdgcn_readlane(slot, G::kRowsPerLoad * q + r);
                s = sub == r ? sr : s;
            }
            row = (uint64_t)row_ptr(vb, v_ss, s);
        }
        rv[q] = ldg16<u32x4_t>((const char *)row + byte_in_row);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Where tile row r of V sits in the wave's LDS tile, in rows of kVPitch.
// The transposed reads of P.V take rows 4j..4j+3 for lane groups j = 0, 1
// together (then j = 2, 3), 32 bytes of each row: those 8 rows must start
// in 8 different 8-bank windows.  The 544-byte pitch (8 banks per row) does
// that in order.  The 528-byte pitch of the 8-query-row layout (4 banks per
// row, which its LDS budget requires) would put rows 0..7 in overlapping
// windows, two lanes per bank; rows 0..7 therefore take the even places and
// rows 8..15 the odd ones, 8 banks apart.  (Counters on the FP8 long prefill
// before this: 48% of the LDS's active cycles stalled on bank conflicts.)
template <int kVPitch>
__device__ __forceinline__ constexpr int v_row(int r) {
    static_assert(kVPitch == kRowBytes + 32 || kVPitch == kRowBytes + 16, "V pitch");
    return kVPitch == kRowBytes + 32 ? r : (((r & 7) << 1) | (r >> 3));
}

// FP8 V rows in LDS (as BF16): a lane converts 16 consecutive dims, 32
// bytes, and writes them as two 16-byte halves.  Written side by side, the 16
// lanes of a row would hit each bank twice (32-byte stride); instead the
// first halves of the row's 16 chunks go to bytes [0, 256) and the second
// halves to [kFp8VHalf, kFp8VHalf + 256), each write contiguous.  Dim d then
// sits at byte ((d % 16) / 8) * kFp8VHalf + 16 (d / 16) + 2 (d % 8); the
// 16-byte gap keeps the transposed reads of the two halves 4 banks apart.
constexpr int kFp8VHalf = 272;
static_assert(kFp8VHalf + 256 <= kRowBytes + 16, "FP8 V row within its pitch");

// Write a gathered V tile into the wave's LDS tile as BF16 rows.
template <KvType KV, int kVPitch>
__device__ __forceinline__ void stage_v(const u32x4_t (&rv)[KvGather<KV>::kVLoads], char *vs,
                                        int lane) {
    using G = KvGather<KV>;
    const int chunk = lane % G::kLanesPerRow;
    const int sub = lane / G::kLanesPerRow;
#pragma unroll
    for (int q = 0; q < G::kVLoads; ++q) {
        const int r = v_row<kVPitch>(G::kRowsPerLoad * q + sub);
        if constexpr (KV == KvType::kBf16) {
            *LDS_PTR(u32x4_t, vs + r * kVPitch + 16 * chunk) = rv[q];
        } else {
            *LDS_PTR(bf16x8_t, vs + r * kVPitch + 16 * chunk) = fp8x8_to_bf16(rv[q][0], rv[q][1]);
            *LDS_PTR(bf16x8_t, vs + r * kVPitch + kFp8VHalf + 16 * chunk) =
                fp8x8_to_bf16(rv[q][2], rv[q][3]);
        }
    }
}


// List entry of tile row (lane & 15) for tile `tile`: -1 for the padding of
// the last tile, 0 for a tile past the list (a prefetch that is never used).
__device__ __forceinline__ int tile_slot(const int32_t *list, int tile, int ntiles, int lane) {
    return tile < ntiles ? list[tile * kTileSlots + (lane & 15)] : 0;
}

// The slot a tile row gathers, from its tile_slot entry: padding rows take
// the tile's first slot (row 0, held by lane 0; valid whenever the tile is
// in the list), so every gather reads a row of the cache and is issued
// unconditionally, with no select on the row address.  The scores of such
// rows are masked to -inf, so their softmax weights are exactly zero and what
// they read never reaches the output.  Called with all lanes active (the
// lane-0 read must not run under a mask of the padding lanes), and where the
// entry was loaded a tile earlier, so it waits for nothing recent.
__device__ __forceinline__ int stand_in(int entry) {
    const int first = max(__builtin_amdgcn_readfirstlane(entry), 0);
    return entry >= 0 ? entry : first;
}

// Masked rows (raw selection rows of decode shares, or aligned block lists):
// the entry of tile row (lane & 15), -1 past the row's n entries, 0 for a tile
// past the row (a prefetch never used).  Each entry names a block of 2^shift
// slots (shift 0: a slot): tile row i reads entry i >> shift.  The loaded
// entry is returned as it is: nothing may compute on it here, or the wave
// would wait for the load (and, loads completing in order, for every gather
// issued before it) at once; block_slot expands it a tile later.
__device__ __forceinline__ int tile_entry_masked(const int32_t *row, int tile, int ntiles, int n,
                                                 int shift, int lane) {
    const int i = tile * kTileSlots + (lane & 15);
    const int e = i >> shift;
    return tile < ntiles ? (e < n ? row[e] : -1) : 0;
}

// The slot tile row (lane & 15) of tile `tile` gathers for entry b of a
// masked list of 2^shift-slot blocks: (b << shift) + the row's offset in its
// block; -1 and other negative entries stay as they are.
__device__ __forceinline__ int block_slot(int b, int tile, int shift, int lane) {
    const int i = tile * kTileSlots + (lane & 15);
    return b >= 0 ? (b << shift) | (i & ((1 << shift) - 1)) : b;
}

// stand_in for masked rows: valid entries (in [0, S)) keep their slot; the
// others read the tile's first valid slot, or slot 0 when it has none.  Also
// returns the tile's valid-row mask (bit r for tile row r) and its count of
// invalid entries other than -1.  Called with every lane active.
__device__ __forceinline__ int stand_in_masked(int entry, int64_t S, uint32_t *valid_rows,
                                               int *n_bad) {
    const bool valid = entry >= 0 && entry < S;
    const uint32_t vm = (uint32_t)(__ballot(valid) & 0xffffu);
    *valid_rows = vm;
    *n_bad = __popcll(__ballot(!valid && entry != -1) & 0xffffu);
    const int first = vm ? __builtin_amdgcn_readlane(entry, __builtin_ctz(vm)) : 0;
    return valid ? entry : first;
}

// ---------------------------------------------------------------- attention

// One wave per workgroup and per work item.
// kSplit = false: the wave takes all tiles of its item and writes BF16.
// kSplit = true: workgroup = (item, split s); it takes tiles s, s + splits,
// s + 2 splits, ... and writes FP32 (O, m, l) of that share to part
// part_base + s, for qsa_merge_partials (or another shard's partials) to
// combine.
//
// Per tile: the score MFMAs consume K(i) from registers; the softmax runs;
// V(i) is written from registers to the wave's LDS tile and the loads of
// V(i+1) are issued one by one; P.V reads V(i) back with transpose loads.
// The loads of K(i+1) go into K(i)'s registers once the scores are done:
// spread over the P.V MFMAs for BF16, around the softmax for FP8.  So about
// one tile of K and V (16 KiB in BF16) is in flight per wave throughout, and
// the wave's requests reach the memory system spread out.  Each wave walks
// its own item's slot list in order, and the list is grouped by slot range,
// so a wave's consecutive tiles fall in the same part of the cache.
//
// kMasked: a row's entries outside [0, S) (-1 included) may stand anywhere in
// it; each tile masks them with a ballot of its rows.  Split shares then read
// the raw selection rows (W_raw entries each); unsplit items read a
// compacted list with -1 gaps (count[t] entries, the aligned block lists).
//
// kKeysLds (BF16, general layout, compacted lists): the keys are gathered
// like the values, as whole rows, two per load instruction, a whole tile
// ahead: at the start of each tile K(i) goes from its registers into the
// wave's LDS tile, the gathers of K(i+1) are issued into those registers at
// once, and the score MFMAs read their K operands back from LDS with the
// same dims per lane as the direct form, so both give the same bits.  The
// values then overwrite the tile as usual.
template <bool kSplit, KvType KV, int kQRows, int kItems, bool kMasked, bool kKeysLds>
__device__ __forceinline__ void attend_unit(const AttendParams &p, const int64_t unit,
                                            char *smem) {
    using Gth = KvGather<KV>;
    using Lay = AttendLayout<kQRows, kItems>;
    constexpr bool kRawRows = kMasked && kSplit;
    static_assert(!kKeysLds || (KV == KvType::kBf16 && kQRows == 16 && !kMasked),
                  "keys through LDS: BF16 general layout over compacted lists");

    int lane = threadIdx.x;
    // In the unit loop of a persistent layout, the lane index is made opaque,
    // so that nothing derived from it is hoisted out of the loop and held
    // across the tile loop (at 4 items per CU: 160 VGPRs instead of 188).
    if constexpr (Lay::kPersistent) asm volatile("" : "+v"(lane));
    const int c = lane & 15;   // MFMA column: query head within the block / A-operand row
    const int j = lane >> 4;   // MFMA lane group

    const int splits = kSplit ? p.splits : 1;
    const int64_t item = kSplit ? unit / splits : unit;
    const int split = kSplit ? (int)(unit - item * splits) : 0;
    const int64_t per_t = (int64_t)p.Hkv * p.HB;
    const int64_t t = item / per_t;
    const int rem = (int)(item - t * per_t);
    const int g = rem / p.HB;
    const int hb = rem - g * p.HB;
    const int h0 = g * p.G + hb * kHeadBlock;
    const int nh = min(kHeadBlock, p.G - hb * kHeadBlock);
    // Entries of the item's row: the compacted list's count, or (raw rows)
    // the selection width, -1 and invalid entries included.  Lists compacted
    // for more cache slots than the views hold are refused: the item reads
    // nothing (a zero row, or an empty share) and flags the workspace.
    // Masked lists count entries of 2^shift slots each (micro-blocks).
    const int shift = kMasked && !kRawRows ? p.block_shift : 0;
    int n_entries;
    if constexpr (kRawRows) {
        n_entries = p.W_raw;
    } else {
        const int cnt = p.count[t];
        const bool fits = (int64_t)p.extent[0] <= p.S_rows;
        n_entries = fits ? cnt : 0;
        if (!fits && lane == 0) p.extent[1] = 1;
    }
    const int n = n_entries << shift;   // slots of the row, gaps included

    const int ntiles = (n + kTileSlots - 1) / kTileSlots;
    // Raw rows: the share of (g = 0, head block 0) reports the invalid entries.
    const bool report_bad = kRawRows && g == 0 && hb == 0;
    const int64_t part_row = kSplit ? ((p.part_base + split) * p.T + t) * p.Hq + h0 : 0;
    if (kSplit && split >= ntiles) {
        // This share is empty: max -inf, sum 0, O 0.
        for (int idx = lane; idx < nh * (kHeadDim / 4); idx += 64) {
            const int hh = idx / (kHeadDim / 4), q4 = idx % (kHeadDim / 4);
            *(f32x4_t *)(p.part_o + (part_row + hh) * kHeadDim + 4 * q4) =
                f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (lane < nh) {
            p.part_ml[(part_row + lane) * 2] = kNegInf;
            p.part_ml[(part_row + lane) * 2 + 1] = 0.0f;
        }
        if (report_bad && lane == 0) p.bad_part[split * p.T + t] = 0;
        return;
    }
    uint16_t *out_t = kSplit ? nullptr : p.out + t * p.o_st + (int64_t)h0 * p.o_sh;
    if (!kSplit && n == 0) {
        // Nothing selected: the output row is exactly +0.0.
        for (int idx = lane; idx < nh * kChunksPerRow; idx += 64) {
            const int hh = idx / kChunksPerRow, ch = idx % kChunksPerRow;
            *(u32x4_t *)(out_t + hh * p.o_sh + ch * 8) = u32x4_t{0, 0, 0, 0};
        }
        return;
    }

    const int32_t *list = kRawRows ? p.raw + t * p.raw_stride : p.list + t * p.list_stride;
    // The next list entries of this lane's tile row (compacted list or raw row).
    auto entry_at = [&](int tl) {
        return kMasked ? tile_entry_masked(list, tl, ntiles, n_entries, shift, lane)
                       : tile_slot(list, tl, ntiles, lane);
    };
    // Tiles of gathers in flight per wave (the layout's; two measured slower
    // for the decode step's split shares too: 25.4 against 24.6 us at 8
    // items per CU, 23.2 against 22.5 at 4).
    constexpr int kAhead = Lay::kAhead;
    // Masked rows: the valid-row mask and invalid count of the tile being
    // computed (cur) and of the tiles whose gathers are in flight, one per
    // register buffer (q).
    uint32_t valid_cur = 0xffffu, valid_q[kAhead];
    int bad_q[kAhead], bad_total = 0;
#pragma unroll
    for (int b = 0; b < kAhead; ++b) {
        valid_q[b] = 0xffffu;
        bad_q[b] = 0;
    }
    // The slot a tile row gathers, from its list entry (loaded a tile
    // earlier) and the tile's index; masked rows record the tile's mask in
    // register buffer b.
    auto resolve = [&](int entry, int tl, int b) {
        if constexpr (kMasked)
            return stand_in_masked(block_slot(entry, tl, shift, lane), p.S_rows, &valid_q[b],
                                   &bad_q[b]);
        else return stand_in(entry);
    };
    const char *kb = (const char *)p.k + (int64_t)g * p.k_sh * Gth::kElemBytes;
    const char *vb = (const char *)p.v + (int64_t)g * p.v_sh * Gth::kElemBytes;
    const uint32_t k_ss = (uint32_t)(p.k_ss * Gth::kElemBytes);
    const uint32_t v_ss = (uint32_t)(p.v_ss * Gth::kElemBytes);
    char *vs_lds = smem;
    char *q_lds = smem + Lay::kTileBytes;

    // The item's query rows (16 heads; absent heads are zero) go to LDS; their
    // loads are issued before the first gathers and written after them.  With
    // the keys through LDS, each lane instead keeps its own query operands of
    // all k-steps in registers (32 more VGPRs; the tiles then read only K and
    // V from LDS: 3.8% faster on the two-request prefill, no change for the
    // direct form, slightly slower at 4 items per CU).
    constexpr bool kQRegs = kKeysLds;
    bf16x8_t qk[kQRegs ? kKSteps : 1];
    if constexpr (kQRegs) {
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const uint16_t *src = c < nh ? p.q + t * p.q_st + (int64_t)(h0 + c) * p.q_sh +
                                               8 * q_chunk(ks, j)
                                         : kZeroRow + 8 * q_chunk(ks, j);
            qk[ks] = ldg16<bf16x8_t>(src);
        }
    }
    u32x4_t qr[Lay::kQChunksPerLane];
#pragma unroll
    for (int u = 0; u < (kQRegs ? 0 : Lay::kQChunksPerLane); ++u) {
        const int idx = lane + 64 * u;
        const int r = idx / kChunksPerRow, ch = idx % kChunksPerRow;
        const uint16_t *src =
            r < nh ? p.q + t * p.q_st + (int64_t)(h0 + r) * p.q_sh + 8 * ch : kZeroRow + 8 * ch;
        qr[u] = ldg16<u32x4_t>(src);
    }

    // This wave's tiles: split, split + splits, ...  The gathers run one
    // tile ahead: rk and rv hold tile i while tile i+1 is in flight, and
    // slot_next holds the list entries of the next tile to gather (turned
    // into slots by stand_in: the gathers are issued unconditionally, so the
    // loaded registers need no copies).  Each slot
    // vector is loaded before the V gathers of the tile ahead of it, so
    // waiting for it never waits for those.  (Two tiles ahead measured no
    // faster.)
    // V row addresses in scalar registers for BF16 at 8 items per CU (the
    // vector form measured 4% slower there: its 64-bit multiplies take vector
    // issue slots); in vector registers for the FP8 layout (12 items per CU,
    // whose waves share the scalar unit of the CU) and at 4 items per CU,
    // where the vector form measured 2-5% faster.
    constexpr bool kScalarVAddr = KV == KvType::kBf16 && Lay::kItems == 8;
    // Wave priority (BF16 keys straight into the MFMA operands): the wave
    // computing its scores, softmax and P.V, with the next tile's K gathers
    // spread over the P.V, takes issue priority over the waves of its SIMD
    // that stage V and issue the next tile's whole-row V gathers.  The V
    // gathers of the waves then reach the memory system at the pace of the
    // others' arithmetic rather than in bursts: long prefill 2.36 against
    // 2.43 ms per step.  The whole-row K gathers of the keys-through-LDS form
    // and the FP8 tiles measured slower this way (two requests 2.12 against
    // 1.98 ms with the priority held over those K gathers), and a priority
    // raised over the V gathers instead made the long prefill 17% slower.
    constexpr bool kPrio = KV == KvType::kBf16 && !kKeysLds;
    const int step = splits;
    u32x4_t rkb[kAhead][Gth::kKLoads], rvb[kAhead][Gth::kVLoads];
    int tile = split;
    int slot_next = entry_at(tile);
#pragma unroll
    for (int b = 0; b < kAhead; ++b) {
        const int slot = resolve(slot_next, tile + b * step, b);
        if constexpr (kKeysLds) gather_v<KV, kScalarVAddr>(rkb[b], slot, kb, k_ss, lane);
        else gather_k<KV>(rkb[b], slot, kb, k_ss, lane);
        slot_next = entry_at(tile + (b + 1) * step);
        gather_v<KV, kScalarVAddr>(rvb[b], slot, vb, v_ss, lane);
    }

#pragma unroll
    for (int u = 0; u < (kQRegs ? 0 : Lay::kQChunksPerLane); ++u) {
        const int idx = lane + 64 * u;
        *LDS_PTR(u32x4_t, q_lds + (idx / kChunksPerRow) * kQPitch + 16 * (idx % kChunksPerRow)) =
            qr[u];
    }
    wave_lds_fence();

    float m = kNegInf;   // running max (log2 domain) for head c
    float lsum = 0.0f;   // this lane's share of the softmax denominator
    f32x4_t o[kDimBlocks];
#pragma unroll
    for (int db = 0; db < kDimBlocks; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // V row this lane addresses in a transpose load (its place in the tile)
    const int tr_row = v_row<Lay::kVPitch>(4 * j + (c >> 2));
    const int tr_sub = c & 3;               // which 4 of the 16 dims of a block
    // Byte offset of those 4 dims within dim block 0 of a row (FP8 rows: the
    // split layout of stage_v; dim block db adds 16 db there, 32 db for BF16).
    const int tr_off = KV == KvType::kFp8 ? (tr_sub >> 1) * kFp8VHalf + 8 * (tr_sub & 1)
                                          : 8 * tr_sub;
    constexpr int kTrBlock = KV == KvType::kFp8 ? 16 : 32;

    // One tile: consumes K(tile) and V(tile) from rk and rv and issues the
    // gathers of tile + kAhead * step into the same registers.
    auto tile_body = [&](const int tile, u32x4_t (&rk)[Gth::kKLoads],
                         u32x4_t (&rv)[Gth::kVLoads], const int b) {
        // S^T for the tile: s[i] = score of tile slot 4j+i against head c.
        // The query operands are read from LDS in two halves to bound the
        // registers they hold (with the keys through LDS they stay in
        // registers, and the K operands come from the tile instead).
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
        int slot_g = 0;   // slots of the tile whose gathers go out next
        bf16x8_t ka[kKeysLds ? kKSteps : 1];
        if constexpr (kKeysLds) {
            wave_lds_fence();   // the previous tile's transpose reads are done
            stage_v<KV, Lay::kVPitch>(rk, vs_lds, lane);   // K(i) rows into the tile
            __builtin_amdgcn_sched_barrier(0);
            slot_g = resolve(slot_next, tile + kAhead * step, b);
            gather_v<KV, kScalarVAddr>(rk, slot_g, kb, k_ss, lane);   // K(i+1)
            wave_lds_fence();
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks)
                ka[ks] = *LDS_PTR(bf16x8_t, vs_lds + v_row<Lay::kVPitch>(c) * Lay::kVPitch +
                                                16 * q_chunk(ks, j));
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8_t qb[kKSteps / 2];
#pragma unroll
            for (int u = 0; u < kKSteps / 2; ++u) {
                if constexpr (kQRegs) qb[u] = qk[(half * kKSteps / 2 + u) % (kQRegs ? kKSteps : 1)];
                else qb[u] = *LDS_PTR(bf16x8_t,
                                      q_lds + (c % kQRows) * kQPitch +
                                          16 * q_chunk(half * kKSteps / 2 + u, j));
            }
#pragma unroll
            for (int u = 0; u < kKSteps / 2; ++u) {
                const int ks = half * kKSteps / 2 + u;
                bf16x8_t kop;
                if constexpr (kKeysLds) kop = ka[ks];
                else kop = k_operand<KV>(rk, ks);
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qb[u], s, 0, 0, 0);
            }
        }
        // Where the loads of the next tile's K go: FP8 tiles are short and
        // latency-bound, so they are issued early, half before the softmax
        // and half after its row maximum; BF16 loads are spread over the P.V
        // MFMAs below, one per two MFMAs (measured fastest of the placements
        // tried: all at once after the scores, spread over the softmax, or
        // alternating with the V loads).  With the keys through LDS they went
        // out as one burst at the start of the tile, above.
        // The next tile's slots: FP8 needs them here; BF16 resolves them after
        // V(i) is staged, where that wait has already covered their load (a
        // resolve here would wait for V(i) before the scores), or, with the
        // keys through LDS, at the start of the tile.
        if constexpr (kMasked) {   // this tile's mask and count, resolved when its gathers went out
            valid_cur = valid_q[b];
            bad_total += bad_q[b];
        }
        if constexpr (KV == KvType::kFp8) slot_g = resolve(slot_next, tile + kAhead * step, b);
        __builtin_amdgcn_sched_barrier(0);   // K(i) is consumed before K(i+1) lands
        if constexpr (KV == KvType::kFp8) {
#pragma unroll
            for (int q = 0; q < Gth::kKLoads / 2; ++q) {
                gather_k1<KV>(rk[q], q, slot_g, kb, k_ss, lane);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // Online softmax in the log2 domain; slots at or past n are masked.
        const int first = tile * kTileSlots + 4 * j;
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool keep = kMasked ? ((valid_cur >> (4 * j + i)) & 1u) != 0 : first + i < n;
            x[i] = keep ? s[i] * p.scale_log2e : kNegInf;
        }
        float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mt = max_over_lane_groups(mt);
        if constexpr (KV == KvType::kFp8) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = Gth::kKLoads / 2; q < Gth::kKLoads; ++q) {
                gather_k1<KV>(rk[q], q, slot_g, kb, k_ss, lane);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const bool raise = mt > m + kRescaleSlack;
        const float m_new = raise ? mt : m;
        if (__ballot(raise)) {
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < kDimBlocks; ++db) o[db] *= alpha;
        }
        m = m_new;
        bf16x4_t pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // (Masked rows: a tile with no valid row, before any valid one,
            // has m = -inf and x = -inf, whose difference is not a number.)
            const __bf16 pr = (kMasked && valid_cur == 0)
                                  ? (__bf16)0.0f
                                  : (__bf16)__builtin_amdgcn_exp2f(x[i] - m);
            pb[i] = pr;
            lsum += (float)pr;
        }

        if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
        wave_lds_fence();   // the previous tile's transpose reads are done
        stage_v<KV, Lay::kVPitch>(rv, vs_lds, lane);
        __builtin_amdgcn_sched_barrier(0);   // V(i) is consumed before V(i+1) lands
        if constexpr (KV == KvType::kBf16 && !kKeysLds)
            slot_g = resolve(slot_next, tile + kAhead * step, b);
        slot_next = entry_at(tile + (kAhead + 1) * step);
        gather_v<KV, kScalarVAddr>(rv, slot_g, vb, v_ss, lane);
        wave_lds_fence();   // other lanes of this wave wrote the rows read below

        if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
        // O^T += V^T . P^T over the tile's 16 slots.  The k index of lane
        // group j is slots 4j..4j+3, matching pb.  ds_read_b64_tr_b16: lane i
        // of a 16-lane group addresses row 4j + i/4, dims 16 db + 4 (i%4);
        // lane c then receives V[4j + e][16 db + c] for e = 0..3.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x4_t va[kDimBlocks / 2];
#pragma unroll
            for (int u = 0; u < kDimBlocks / 2; ++u) {
                const int db = half * (kDimBlocks / 2) + u;
                va[u] = __builtin_bit_cast(
                    bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(
                                  i16x4_t, vs_lds + tr_row * Lay::kVPitch + kTrBlock * db + tr_off)));
            }
#pragma unroll
            for (int u = 0; u < kDimBlocks / 2; ++u) {
                const int db = half * (kDimBlocks / 2) + u;
                o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[u], pb, o[db], 0, 0, 0);
                constexpr int kEvery = kDimBlocks / Gth::kKLoads;
                if (KV == KvType::kBf16 && !kKeysLds && db % kEvery == kEvery - 1) {
                    __builtin_amdgcn_sched_barrier(0);
                    gather_k1<KV>(rk[db / kEvery], db / kEvery, slot_g, kb, k_ss, lane);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };
    for (; tile < ntiles; tile += kAhead * step) {
#pragma unroll
        for (int b = 0; b < kAhead; ++b) {
            if (b > 0 && tile + b * step >= ntiles) break;
            tile_body(tile + b * step, rkb[b], rvb[b], b);
            if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
        }
    }

    // Whole-head denominator: add the four lane groups.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    // Lane (c, j) holds dims 16 db + 4 j .. +4 of head c.
    if (c < nh) {
        if (kSplit && j == 0) {
            p.part_ml[(part_row + c) * 2] = m;
            p.part_ml[(part_row + c) * 2 + 1] = lsum;
        }
        if (report_bad && lane == 0) p.bad_part[split * p.T + t] = bad_total;
#pragma unroll
        for (int db = 0; db < kDimBlocks; ++db) {
            f32x4_t acc = o[db];
            if constexpr (KV == KvType::kFp8) acc *= p.v_scale;
            if (kSplit) {
                *(f32x4_t *)(p.part_o + (part_row + c) * kHeadDim + 16 * db + 4 * j) = acc;
            } else {
                bf16x4_t ob;
#pragma unroll
                for (int i = 0; i < 4; ++i) ob[i] = (__bf16)(acc[i] / lsum);
                *(u32x2_t *)(out_t + (int64_t)c * p.o_sh + 16 * db + 4 * j) =
                    __builtin_bit_cast(u32x2_t, ob);
            }
        }
    }
}

// One workgroup per work unit; or, for a persistent layout, at most one
// chip-full of workgroups, workgroup w taking units w, w + grid, w + 2 grid,
// ... (the grid is a multiple of the 8 XCDs, so unit u still runs on XCD
// u % 8).  Persistent workgroups measured 1.5-2% faster at 4 items per CU
// and 2.5-4% slower at 8 and 12, where the hardware's refill of finished
// workgroups keeps the running tokens closer together.
template <bool kSplit, KvType KV, int kQRows, int kItems = kItemsPerCU, bool kMasked = false,
          bool kKeysLds = false>
__global__ __launch_bounds__(64, (AttendLayout<kQRows, kItems>::kWavesPerSimd)) void attend_kernel(
    const AttendParams p) {
    using Lay = AttendLayout<kQRows, kItems>;
    __shared__ __attribute__((aligned(16))) char smem[Lay::kLds];
    if (p.choice != nullptr && *p.choice != p.choice_value) return;
    if constexpr (Lay::kPersistent) {
        for (int64_t unit = blockIdx.x; unit < p.units; unit += gridDim.x) {
            wave_lds_fence();   // the previous unit's LDS reads are done
            attend_unit<kSplit, KV, kQRows, kItems, kMasked, kKeysLds>(p, unit, smem);
        }
    } else {
        attend_unit<kSplit, KV, kQRows, kItems, kMasked, kKeysLds>(p, blockIdx.x, smem);
    }
}

// ---------------------------------------------------------------- merge

// out[t, h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the parts s,
// M = max_s m_s; exactly +0.0 when no part saw a slot.  One 256-thread
// workgroup per (t, h) row, 4 dims per lane: wave w takes the parts
// s = w + 4 j.  A wave issues the O loads of its first kMergeBatch parts
// together with the (m, l) loads (they do not depend on M), so up to 32
// parts arrive in one memory round trip; the four waves then exchange
// their maxima and their weighted sums through LDS, added in wave order.
// (One wave per row, its parts read 8 at a time, took 6.4 us on the decode
// step: four dependent round trips.)
constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 8;

__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
    __shared__ float wave_m[kMergeWaves], wave_l[kMergeWaves];
    __shared__ f32x4_t wave_acc[kMergeWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = blockIdx.x;   // < T * Hq (the grid)
    const int64_t rows = p.T * p.Hq;
    const int64_t t = row / p.Hq;
    const int h = (int)(row - t * p.Hq);
    const int64_t n = p.n_parts;
    // This wave's parts: s(j) = wave + kMergeWaves j, j < J.
    const int64_t J = n > wave ? (n - wave + kMergeWaves - 1) / kMergeWaves : 0;
    auto o_row = [&](int64_t j) {
        return (const f32x4_t *)(p.part_o + ((wave + kMergeWaves * j) * rows + row) * kHeadDim +
                                 4 * lane);
    };
    if (p.clear_flag != nullptr && row == 0 && threadIdx.x == 0) *p.clear_flag = 0;
    if (p.bad_part != nullptr && h == 0 && wave == 0) {
        // The invalid entries of token t's row, reported by its raw-row shares.
        int bad = 0;
        for (int64_t s = lane; s < n; s += 64) bad += p.bad_part[s * p.T + t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) bad += __shfl_xor(bad, off);
        if (lane == 0) p.n_bad[t] = bad;
    }
    // The first batch of O rows, in flight with the (m, l) loads below.
    f32x4_t o0[kMergeBatch];
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e)
        o0[e] = e < J ? *o_row(e) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_loc = kNegInf;
    for (int64_t j = lane; j < J; j += 64)
        m_loc = fmaxf(m_loc, p.part_ml[((wave + kMergeWaves * j) * rows + row) * 2]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m_loc = fmaxf(m_loc, __shfl_xor(m_loc, off));
    if (lane == 0) wave_m[wave] = m_loc;
    __syncthreads();
    float mmax = wave_m[0];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) mmax = fmaxf(mmax, wave_m[w]);

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float l_part = 0.0f;
    if (mmax != kNegInf) {   // the same for every wave
        for (int64_t j0 = 0; j0 < J; j0 += 64) {
            // Lane j - j0 holds part j's weight.
            float w = 0.0f;
            if (j0 + lane < J) {
                const float *ml = p.part_ml + ((wave + kMergeWaves * (j0 + lane)) * rows + row) * 2;
                w = __builtin_amdgcn_exp2f(ml[0] - mmax);
                l_part += w * ml[1];
            }
            const int cnt = (int)min<int64_t>(64, J - j0);
            for (int u = 0; u < cnt; u += kMergeBatch) {
                f32x4_t o[kMergeBatch];
                if (j0 == 0 && u == 0) {
#pragma unroll
                    for (int e = 0; e < kMergeBatch; ++e) o[e] = o0[e];
                } else {
#pragma unroll
                    for (int e = 0; e < kMergeBatch; ++e)
                        o[e] = u + e < cnt ? *o_row(j0 + u + e) : f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int e = 0; e < kMergeBatch; ++e)
                    if (u + e < cnt)
                        acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u + e)) *
                               o[e];
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) l_part += __shfl_xor(l_part, off);
    wave_acc[wave][lane] = acc;
    if (lane == 0) wave_l[wave] = l_part;
    __syncthreads();
    if (wave == 0) {
        bf16x4_t ob = {(__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
        if (mmax != kNegInf) {
            f32x4_t sum = wave_acc[0][lane];
            float l_tot = wave_l[0];
#pragma unroll
            for (int w = 1; w < kMergeWaves; ++w) {
                sum += wave_acc[w][lane];
                l_tot += wave_l[w];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) ob[i] = (__bf16)(sum[i] / l_tot);
        }
        *(u32x2_t *)(p.out + t * p.o_st + (int64_t)h * p.o_sh + 4 * lane) =
            __builtin_bit_cast(u32x2_t, ob);
    }
}

// Many rows: one wave per row, kMergeRowsPerWg rows per workgroup, no LDS and
// no barrier.  The wave runs merge_kernel's four part sequences s = w + 4 j
// one after the other with the same operations in the same order (weights in
// the lanes of their sequence, weighted O rows added in sequence order,
// denominators reduced across lanes per sequence, the four sums added in
// sequence order), so both kernels give the same bits and the choice between
// them is one of speed only.  merge_kernel spends a workgroup and two barriers
// on each row: on 124,960 rows of one part (the long prefill's rows) it took
// 0.38 ms, about 60 generations of short-lived workgroups; this kernel takes
// 56 us.  Its few loads ahead keep it at 60 VGPRs, 8 waves per SIMD: two rows
// ahead per sequence and batches of four (94 VGPRs) took 77 us.
constexpr int kMergeRowsPerWg = 4;
constexpr int kMergeRowsAhead = 1;   // O rows per sequence loaded with the maxima
constexpr int kMergeRowsBatch = 2;   // O rows per sequence loaded together after that
static_assert(kMergeRowsAhead <= kMergeRowsBatch, "the rows loaded ahead serve the first batch");
// merge_kernel below this many rows (the parts of a row spread over four waves
// keep a decode step's few rows in one memory round trip), this kernel from it.
constexpr int64_t kMergeRowsMin = 4096;

__global__ __launch_bounds__(256) void merge_rows_kernel(const MergeParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t rows = p.T * p.Hq;
    const int64_t row = (int64_t)blockIdx.x * kMergeRowsPerWg + (threadIdx.x >> 6);
    if (row >= rows) return;   // (whole waves; nothing below waits on other waves)
    const int64_t t = row / p.Hq;
    const int h = (int)(row - t * p.Hq);
    const int64_t n = p.n_parts;
    auto o_row = [&](int64_t s) {
        return (const f32x4_t *)(p.part_o + (s * rows + row) * kHeadDim + 4 * lane);
    };
    if (p.clear_flag != nullptr && row == 0 && lane == 0) *p.clear_flag = 0;
    if (p.bad_part != nullptr && h == 0) {
        int bad = 0;
        for (int64_t s = lane; s < n; s += 64) bad += p.bad_part[s * p.T + t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) bad += __shfl_xor(bad, off);
        if (lane == 0) p.n_bad[t] = bad;
    }
    // The first O rows of every sequence, in flight with the maxima.
    f32x4_t o0[kMergeWaves][kMergeRowsAhead];
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w)
#pragma unroll
        for (int e = 0; e < kMergeRowsAhead; ++e) {
            const int64_t s = w + (int64_t)kMergeWaves * e;
            o0[w][e] = s < n ? *o_row(s) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    float mmax = kNegInf;
    for (int64_t s = lane; s < n; s += 64) mmax = fmaxf(mmax, p.part_ml[(s * rows + row) * 2]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, off));

    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
    float l_tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
        const int64_t J = n > w ? (n - w + kMergeWaves - 1) / kMergeWaves : 0;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        float l_part = 0.0f;
        if (mmax != kNegInf) {
            for (int64_t j0 = 0; j0 < J; j0 += 64) {
                // Lane j - j0 holds part w + 4 j's weight.
                float wt = 0.0f;
                if (j0 + lane < J) {
                    const float *ml = p.part_ml + ((w + kMergeWaves * (j0 + lane)) * rows + row) * 2;
                    wt = __builtin_amdgcn_exp2f(ml[0] - mmax);
                    l_part += wt * ml[1];
                }
                const int cnt = (int)min<int64_t>(64, J - j0);
                for (int u = 0; u < cnt; u += kMergeRowsBatch) {
                    f32x4_t o[kMergeRowsBatch];
                    const bool first = j0 == 0 && u == 0;
#pragma unroll
                    for (int e = 0; e < kMergeRowsBatch; ++e) {
                        if (e < kMergeRowsAhead && first)
                            o[e] = o0[w][e < kMergeRowsAhead ? e : 0];
                        else
                            o[e] = u + e < cnt ? *o_row(w + kMergeWaves * (j0 + u + e))
                                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
#pragma unroll
                    for (int e = 0; e < kMergeRowsBatch; ++e)
                        if (u + e < cnt)
                            acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt),
                                                                             u + e)) * o[e];
                }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) l_part += __shfl_xor(l_part, off);
        if (w == 0) {
            sum = acc;
            l_tot = l_part;
        } else {
            sum += acc;
            l_tot += l_part;
        }
    }
    bf16x4_t ob = {(__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
    if (mmax != kNegInf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[i] = (__bf16)(sum[i] / l_tot);
    }
    *(u32x2_t *)(p.out + t * p.o_st + (int64_t)h * p.o_sh + 4 * lane) =
        __builtin_bit_cast(u32x2_t, ob);
}

// ---------------------------------------------------------------- sharing estimate

// One workgroup per sampled token pair (a, b): a's list (at most kShareKeys
// entries of it) goes into a hash set in LDS, b's list is looked up in it.
// The set is kShareBuckets buckets of 8 entries (2 keys per bucket on
// average), filled through per-bucket counters; a key that finds its bucket
// full goes on to the next.  A lookup reads one 32-byte bucket, so every
// lane of a wave finishes in about the same number of steps.  The count of
// common slots, scaled by the share of a's list that was hashed, and |L_b|
// go to est[pair]; sharing_choice_kernel then adds them up and writes the
// choice (see SharingParams).
constexpr int kShareKeys = 2048;
constexpr int kShareBuckets = 1024;
constexpr int kShareBucketSize = 8;

__device__ __forceinline__ uint32_t share_bucket(int32_t key) {
    return ((uint32_t)key * 2654435761u) >> (32 - 10);
}
static_assert(kShareBuckets == 1 << 10, "share_bucket yields 10 bits");

// True if `key` is in bucket bk; *full says whether the bucket has no free
// entry (then a key of this home bucket may have moved on to the next).
__device__ __forceinline__ bool share_in_bucket(const int32_t *table, uint32_t bk, int32_t key,
                                                bool *full) {
    const i32x4_t e0 = *(const i32x4_t *)&table[bk * kShareBucketSize];
    const i32x4_t e1 = *(const i32x4_t *)&table[bk * kShareBucketSize + 4];
    *full = e1[3] != -1;
    return e0[0] == key || e0[1] == key || e0[2] == key || e0[3] == key || e1[0] == key ||
           e1[1] == key || e1[2] == key || e1[3] == key;
}

__global__ __launch_bounds__(256) void sharing_kernel(const SharingParams p) {
    constexpr int kPerThread = kShareKeys / 256;
    __shared__ __attribute__((aligned(16))) int32_t table[kShareBuckets * kShareBucketSize];
    __shared__ int32_t fill[kShareBuckets];
    __shared__ int wave_hits[4];
    const int tid = threadIdx.x;
    const int k = blockIdx.x;
    const int32_t *la = p.list + (int64_t)p.pair_a[k] * p.row_stride;
    const int32_t *lb = p.list + (int64_t)p.pair_b[k] * p.row_stride;
    const int na = p.count[p.pair_a[k]], nb = p.count[p.pair_b[k]];
    // Entry tid + 256 u of each row, all loads in flight at once (rows are
    // row_stride long; entries past a row's count are never used).
    int32_t ka[kPerThread], kb[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        const int i = tid + 256 * u;
        ka[u] = i < p.row_stride ? la[i] : -1;
        kb[u] = i < p.row_stride ? lb[i] : -1;
    }
    for (int i = tid; i < kShareBuckets * kShareBucketSize / 4; i += 256)
        *(i32x4_t *)&table[4 * i] = i32x4_t{-1, -1, -1, -1};
    for (int i = tid; i < kShareBuckets; i += 256) fill[i] = 0;
    __syncthreads();
    // At most kShareKeys keys in kShareBuckets * 8 entries: a free entry is
    // always found.  The home buckets of a thread's keys are claimed
    // together; the rare key whose home bucket is full walks on.
    const int nh = min(na, kShareKeys);
    int pos[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
        pos[u] = tid + 256 * u < nh ? atomicAdd(&fill[share_bucket(ka[u])], 1) : 0;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        if (tid + 256 * u >= nh) continue;
        uint32_t bk = share_bucket(ka[u]);
        int at = pos[u];
        while (at >= kShareBucketSize) {
            bk = (bk + 1) & (kShareBuckets - 1);
            at = atomicAdd(&fill[bk], 1);
        }
        table[bk * kShareBucketSize + at] = ka[u];
    }
    __syncthreads();
    int hits = 0;
    bool found[kPerThread], full[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
        found[u] = share_in_bucket(table, share_bucket(kb[u]), kb[u], &full[u]);
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        if (tid + 256 * u >= nb) continue;
        bool hit = found[u], more = full[u];
        for (uint32_t bk = share_bucket(kb[u]); !hit && more;) {
            bk = (bk + 1) & (kShareBuckets - 1);
            hit = share_in_bucket(table, bk, kb[u], &more);
        }
        hits += hit;
    }
    // Rows longer than kShareKeys entries: the rest of b, one at a time.
#pragma unroll 1
    for (int i = kShareKeys + tid; i < nb; i += 256) {
        const int32_t key = lb[i];
        bool hit = false, more = true;
        for (uint32_t bk = share_bucket(key); !hit && more; bk = (bk + 1) & (kShareBuckets - 1))
            hit = share_in_bucket(table, bk, key, &more);
        hits += hit;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) hits += __shfl_xor(hits, off);
    if ((tid & 63) == 0) wave_hits[tid >> 6] = hits;
    __syncthreads();
    if (tid == 0) {
        const int total = wave_hits[0] + wave_hits[1] + wave_hits[2] + wave_hits[3];
        p.est[2 * k] = nh > 0 ? (float)total * ((float)na / (float)nh) : 0.0f;
        p.est[2 * k + 1] = (float)nb;
    }
}

// One wave: adds up the pairs' counts and writes the choice (the launch
// boundary after sharing_kernel makes its stores visible).
__global__ __launch_bounds__(64) void sharing_choice_kernel(const SharingParams p) {
    const int lane = threadIdx.x;
    float common = 0.0f, len = 0.0f;
    if (lane < p.pairs) {
        common = p.est[2 * lane];
        len = p.est[2 * lane + 1];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        common += __shfl_xor(common, off);
        len += __shfl_xor(len, off);
    }
    if (lane == 0) {
        const float shared = p.lambda_scale * common;
        int choice = 0;
        if (len > 0.0f && shared < p.threshold * len) choice = 1;
        else if (len > 0.0f && p.lds_threshold > 0.0f && shared >= p.lds_threshold * len) choice = 2;
        *p.choice = choice;
    }
}

// ---------------------------------------------------------------- gather only

// Issues the same loads as attend_kernel (same load pattern, tiles, one wave
// per (t, g), same residency per CU) with no arithmetic between them, folds
// them with XOR and writes one word per (t, g).  It shows the cost of the
// gathers issued back to back; the attention kernel, whose work between the
// K and the V loads paces each wave's requests, can run faster than this.
template <KvType KV>
__global__ __launch_bounds__(64, kAttendWavesPerSimd) void gather_only_kernel(const GatherParams p) {
    using Gth = KvGather<KV>;
    // Same LDS footprint as attend_kernel's general layout, so the same number
    // of items fit a CU.
    __shared__ __attribute__((aligned(16))) uint32_t smem[AttendLayout<16>::kLds / 4];
    const int lane = threadIdx.x;
    const int64_t item = blockIdx.x;
    const int64_t t = item / p.Hkv;
    const int g = (int)(item - t * p.Hkv);
    const int cnt = p.count[t];
    // Lists compacted for more slots than the views hold are not read.
    const int n = (int64_t)p.extent[0] <= p.S_rows ? cnt : 0;
    const int ntiles = (n + kTileSlots - 1) / kTileSlots;
    if (ntiles == 0) {   // nothing to read (and maybe no cache row to stand in)
        if (lane == 0) p.sink[item] = 0;
        return;
    }
    const int32_t *list = p.list + t * p.list_stride;
    const char *kb = (const char *)p.k + (int64_t)g * p.k_sh * Gth::kElemBytes;
    const char *vb = (const char *)p.v + (int64_t)g * p.v_sh * Gth::kElemBytes;
    const uint32_t k_ss = (uint32_t)(p.k_ss * Gth::kElemBytes);
    const uint32_t v_ss = (uint32_t)(p.v_ss * Gth::kElemBytes);

    u32x4_t acc = {0, 0, 0, 0};
    u32x4_t rk[Gth::kKLoads], rv[Gth::kVLoads];
    int tile = 0;
    int slot_next;
    {
        const int slot = stand_in(tile_slot(list, tile, ntiles, lane));
        gather_k<KV>(rk, slot, kb, k_ss, lane);
        slot_next = tile_slot(list, tile + 1, ntiles, lane);
        gather_v<KV, KV == KvType::kBf16>(rv, slot, vb, v_ss, lane);
    }
    const u32x4_t zero = {0, 0, 0, 0};
    for (; tile < ntiles; ++tile) {
        // Only the rows of the list are folded (padding rows read stand-ins).
        const int rows = n - tile * kTileSlots;
#pragma unroll
        for (int q = 0; q < Gth::kKLoads; ++q) acc ^= (lane & 15) < rows ? rk[q] : zero;
        const int slot = stand_in(slot_next);
        __builtin_amdgcn_sched_barrier(0);
        gather_k<KV>(rk, slot, kb, k_ss, lane);
#pragma unroll
        for (int q = 0; q < Gth::kVLoads; ++q)
            acc ^= Gth::kRowsPerLoad * q + lane / Gth::kLanesPerRow < rows ? rv[q] : zero;
        __builtin_amdgcn_sched_barrier(0);
        slot_next = tile_slot(list, tile + 2, ntiles, lane);
        gather_v<KV, KV == KvType::kBf16>(rv, slot, vb, v_ss, lane);
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
    // Every lane holds the fold; it reaches lane 0 through the LDS block (from
    // lane 63), which keeps the block allocated.
    smem[lane] = x;
    wave_lds_fence();
    if (lane == 0) p.sink[item] = smem[63];
}

}  // namespace

int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kXcds * kCusPerXcd;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = kXcds * kCusPerXcd;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// attend_kernel over `units` work units: one workgroup each, or at most one
// chip-full (a multiple of the XCDs) for a persistent layout.
template <bool kSplit, KvType KV, int kQRows, int kItems = kItemsPerCU, bool kMasked = false,
          bool kKeysLds = false>
void launch_attend_kernel(AttendParams p, int64_t units, hipStream_t stream) {
    using Lay = AttendLayout<kQRows, kItems>;
    p.units = units;
    int64_t grid = units;
    if (Lay::kPersistent) {
        const int64_t full = std::max<int64_t>(
            kXcds, (int64_t)Lay::kItems * device_cus() / kXcds * kXcds);
        grid = std::min(units, full);
    }
    hipLaunchKernelGGL((attend_kernel<kSplit, KV, kQRows, kItems, kMasked, kKeysLds>),
                       dim3((unsigned)grid), dim3(64), 0, stream, p);
}

// FP8 caches with at most 8 query heads per KV head take the 8-query-row
// layout (12 items per CU); everything else the general one.
template <bool kSplit>
void launch_attend_any(const AttendParams &p, KvType kv, int64_t blocks, hipStream_t stream) {
    if (kv == KvType::kFp8 && p.G <= 8)
        launch_attend_kernel<kSplit, KvType::kFp8, 8>(p, blocks, stream);
    else if (kv == KvType::kFp8)
        launch_attend_kernel<kSplit, KvType::kFp8, 16>(p, blocks, stream);
    else
        launch_attend_kernel<kSplit, KvType::kBf16, 16>(p, blocks, stream);
}

hipError_t launch_attend(const AttendParams &p, KvType kv, int64_t T, hipStream_t stream,
                         const SharingParams *share) {
    const int64_t items = T * (int64_t)p.Hkv * p.HB;
    if (items == 0) return hipSuccess;
    if (p.masked) {   // aligned block lists: BF16, the general layout
        if (kv != KvType::kBf16 || share != nullptr) return hipErrorInvalidValue;
        launch_attend_kernel<false, KvType::kBf16, 16, kItemsPerCU, true>(p, items, stream);
        return hipGetLastError();
    }
    if (share == nullptr && p.keys_lds && kv == KvType::kBf16) {
        launch_attend_kernel<false, KvType::kBf16, 16, kItemsPerCU, false, true>(p, items, stream);
        return hipGetLastError();
    }
    if (share == nullptr || (kv == KvType::kFp8 && p.G <= 8)) {
        launch_attend_any<false>(p, kv, items, stream);
        return hipGetLastError();
    }
    // The estimate picks one of the gated launches of the general layout (8
    // items per CU; 4; BF16: 8 with keys through LDS); the others return at
    // once.  All compute the same bits.
    hipLaunchKernelGGL(sharing_kernel, dim3((unsigned)share->pairs), dim3(256), 0, stream, *share);
    hipLaunchKernelGGL(sharing_choice_kernel, dim3(1), dim3(64), 0, stream, *share);
    AttendParams g = p;
    g.choice = share->choice;
    g.choice_value = 0;
    if (kv == KvType::kFp8)
        launch_attend_kernel<false, KvType::kFp8, 16>(g, items, stream);
    else
        launch_attend_kernel<false, KvType::kBf16, 16>(g, items, stream);
    g.choice_value = 1;
    if (kv == KvType::kFp8)
        launch_attend_kernel<false, KvType::kFp8, 16, kLowShareItemsPerCU>(g, items, stream);
    else
        launch_attend_kernel<false, KvType::kBf16, 16, kLowShareItemsPerCU>(g, items, stream);
    if (kv == KvType::kBf16 && share->lds_threshold > 0.0f) {
        g.choice_value = 2;
        launch_attend_kernel<false, KvType::kBf16, 16, kItemsPerCU, false, true>(g, items, stream);
    }
    return hipGetLastError();
}

hipError_t launch_attend_partial(const AttendParams &p, KvType kv, int64_t T,
                                 hipStream_t stream) {
    const int64_t blocks = T * (int64_t)p.Hkv * p.HB * p.splits;
    if (blocks == 0) return hipSuccess;
    if (p.raw_rows) {   // raw selection rows, masked per tile
        if (p.raw == nullptr && p.W_raw > 0) return hipErrorInvalidValue;
        // The layouts of launch_attend_any, except that BF16 shares take the
        // 4-items-per-CU layout from kDecodeMinUnits units up (decode step of
        // 16 tokens at 16 shares: 21.0 against 22.7 us; 64 tokens at 8 shares:
        // 53.2 against 53.4) and the 8-items one below (1 to 4 tokens at 32
        // shares: 0.2-0.3 us faster).  FP8 caches: the 8-items layouts
        // measured faster (17.1 against 18.1 us on the 16-token step).
        if (kv == KvType::kFp8 && p.G <= 8)
            launch_attend_kernel<true, KvType::kFp8, 8, kItemsPerCU, true>(p, blocks, stream);
        else if (kv == KvType::kFp8)
            launch_attend_kernel<true, KvType::kFp8, 16, kItemsPerCU, true>(p, blocks, stream);
        else if (blocks >= kDecodeMinUnits)
            launch_attend_kernel<true, KvType::kBf16, 16, kLowShareItemsPerCU, true>(p, blocks,
                                                                                      stream);
        else
            launch_attend_kernel<true, KvType::kBf16, 16, kItemsPerCU, true>(p, blocks, stream);
        return hipGetLastError();
    }
    launch_attend_any<true>(p, kv, blocks, stream);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeParams &p, hipStream_t stream) {
    const int64_t rows = p.T * p.Hq;
    if (rows == 0) return hipSuccess;
    if (rows >= kMergeRowsMin)
        hipLaunchKernelGGL(merge_rows_kernel,
                           dim3((unsigned)((rows + kMergeRowsPerWg - 1) / kMergeRowsPerWg)),
                           dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(merge_kernel, dim3((unsigned)rows), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_gather_only(const GatherParams &p, KvType kv, int64_t T, hipStream_t stream) {
    const int64_t items = T * (int64_t)p.Hkv;
    if (items == 0) return hipSuccess;
    if (kv == KvType::kFp8)
        hipLaunchKernelGGL(gather_only_kernel<KvType::kFp8>, dim3((unsigned)items), dim3(64), 0,
                           stream, p);
    else
        hipLaunchKernelGGL(gather_only_kernel<KvType::kBf16>, dim3((unsigned)items), dim3(64), 0,
                           stream, p);
    return hipGetLastError();
}

}  // namespace qsa
