// HIP kernels for QSA sparse main-attention prefill on gfx950 (MI355X, CDNA4).
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
//     writes the row in BF16.  Its split form writes FP32 (O, m, l) partials
//     of a share of the tiles instead, which merge_kernel combines.
// Also here: gather_only_kernel (the attention's loads alone, a measurement
// aid), and the QSA indexer that produces the selection: indexer_scores_kernel
// (index scores with bf16 MFMA) and the Top-K selection kernels.

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

#include <hipcub/block/block_load.hpp>
#include <hipcub/block/block_radix_sort.hpp>
#include <hipcub/block/block_reduce.hpp>
#include <hipcub/block/block_scan.hpp>

#include "qsa_kernels.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))
#define GLOBAL_PTR(T, p) ((const __attribute__((address_space(1))) T *)(p))

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
constexpr float kNegInf = -__builtin_huge_valf();
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

// A row of zeros: absent query heads (and index rows past the end) load from
// here, so every load is unconditional and no select waits on loaded data.
__device__ __attribute__((aligned(16))) uint16_t kZeroRow[kHeadDim] = {};

// 16-byte load through the global address space (all operands of the
// gathers, including kZeroRow, are global memory; a generic pointer would
// turn the loads into flat loads).
template <typename V>
__device__ __forceinline__ V ldg16(const void *p) {
    return *GLOBAL_PTR(V, p);
}

// ---------------------------------------------------------------- compaction

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

// ---------------------------------------------------------------- gathers

// Start of the cache row of `slot` (a valid slot: see stand_in).
__device__ __forceinline__ const char *row_ptr(const char *base, int64_t ss, int slot) {
    return base + (int64_t)slot * ss;
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
                                          int64_t k_ss, int lane) {
    const int j = lane >> 4;
    const char *row = row_ptr(kb, k_ss, slot);
    if constexpr (KV == KvType::kBf16)
        r = ldg16<u32x4_t>(row + 128 * (q >> 1) + 32 * j + 16 * (q & 1));
    else
        r = ldg16<u32x4_t>(row + 64 * q + 16 * j);
}

template <KvType KV>
__device__ __forceinline__ void gather_k(u32x4_t (&rk)[KvGather<KV>::kKLoads], int slot,
                                         const char *kb, int64_t k_ss, int lane) {
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
                                         const char *vb, int64_t v_ss, int lane) {
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

// Write a gathered V tile into the wave's LDS tile as BF16 rows.
template <KvType KV, int kVPitch>
__device__ __forceinline__ void stage_v(const u32x4_t (&rv)[KvGather<KV>::kVLoads], char *vs,
                                        int lane) {
    using G = KvGather<KV>;
    const int chunk = lane % G::kLanesPerRow;
    const int sub = lane / G::kLanesPerRow;
#pragma unroll
    for (int q = 0; q < G::kVLoads; ++q) {
        const int r = G::kRowsPerLoad * q + sub;
        if constexpr (KV == KvType::kBf16) {
            *LDS_PTR(u32x4_t, vs + r * kVPitch + 16 * chunk) = rv[q];
        } else {
            *LDS_PTR(bf16x8_t, vs + r * kVPitch + 32 * chunk) = fp8x8_to_bf16(rv[q][0], rv[q][1]);
            *LDS_PTR(bf16x8_t, vs + r * kVPitch + 32 * chunk + 16) =
                fp8x8_to_bf16(rv[q][2], rv[q][3]);
        }
    }
}

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
// entry of tile row (lane & 15), -1 past the row's W entries, 0 for a tile
// past the row (a prefetch never used).
__device__ __forceinline__ int tile_entry_masked(const int32_t *row, int tile, int ntiles, int W,
                                                 int lane) {
    const int i = tile * kTileSlots + (lane & 15);
    return tile < ntiles ? (i < W ? row[i] : -1) : 0;
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
template <bool kSplit, KvType KV, int kQRows, int kItems, bool kMasked>
__device__ __forceinline__ void attend_unit(const AttendParams &p, const int64_t unit,
                                            char *smem) {
    using Gth = KvGather<KV>;
    using Lay = AttendLayout<kQRows, kItems>;
    static_assert(!kMasked || Lay::kAhead == 1, "masked rows: one tile ahead");
    constexpr bool kRawRows = kMasked && kSplit;

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
    // the selection width, -1 and invalid entries included.
    const int n = kRawRows ? p.W_raw : p.count[t];

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
        return kMasked ? tile_entry_masked(list, tl, ntiles, n, lane) : tile_slot(list, tl, ntiles, lane);
    };
    // Masked rows: the valid-row mask and invalid count of the tile being
    // computed (cur) and of the tile whose gathers were issued last (next).
    uint32_t valid_cur = 0xffffu, valid_next = 0xffffu;
    int bad_next = 0, bad_total = 0;
    auto resolve = [&](int entry) {
        if constexpr (kMasked) return stand_in_masked(entry, p.S_rows, &valid_next, &bad_next);
        else return stand_in(entry);
    };
    const char *kb = (const char *)p.k + (int64_t)g * p.k_sh * Gth::kElemBytes;
    const char *vb = (const char *)p.v + (int64_t)g * p.v_sh * Gth::kElemBytes;
    const int64_t k_ss = p.k_ss * Gth::kElemBytes, v_ss = p.v_ss * Gth::kElemBytes;
    char *vs_lds = smem;
    char *q_lds = smem + Lay::kTileBytes;

    // The item's query rows (16 heads; absent heads are zero) go to LDS; their
    // loads are issued before the first gathers and written after them.
    u32x4_t qr[Lay::kQChunksPerLane];
#pragma unroll
    for (int u = 0; u < Lay::kQChunksPerLane; ++u) {
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
    constexpr int kAhead = Lay::kAhead;
    // V row addresses in scalar registers for BF16 at 8 items per CU (the
    // vector form measured 4% slower there: its 64-bit multiplies take vector
    // issue slots); in vector registers for the FP8 layout (12 items per CU,
    // whose waves share the scalar unit of the CU) and at 4 items per CU,
    // where the vector form measured 2-5% faster.
    constexpr bool kScalarVAddr = KV == KvType::kBf16 && Lay::kItems == 8;
    const int step = splits;
    u32x4_t rkb[kAhead][Gth::kKLoads], rvb[kAhead][Gth::kVLoads];
    int tile = split;
    int slot_next = entry_at(tile);
#pragma unroll
    for (int b = 0; b < kAhead; ++b) {
        const int slot = resolve(slot_next);
        gather_k<KV>(rkb[b], slot, kb, k_ss, lane);
        slot_next = entry_at(tile + (b + 1) * step);
        gather_v<KV, kScalarVAddr>(rvb[b], slot, vb, v_ss, lane);
    }

#pragma unroll
    for (int u = 0; u < Lay::kQChunksPerLane; ++u) {
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

    const int tr_row = 4 * j + (c >> 2);    // V row this lane addresses in a transpose load
    const int tr_sub = c & 3;               // which 4 of the 16 dims of a block

    // One tile: consumes K(tile) and V(tile) from rk and rv and issues the
    // gathers of tile + kAhead * step into the same registers.
    auto tile_body = [&](const int tile, u32x4_t (&rk)[Gth::kKLoads],
                         u32x4_t (&rv)[Gth::kVLoads]) {
        // S^T for the tile: s[i] = score of tile slot 4j+i against head c.
        // The query operands are read from LDS in two halves to bound the
        // registers they hold.
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            bf16x8_t qb[kKSteps / 2];
#pragma unroll
            for (int u = 0; u < kKSteps / 2; ++u)
                qb[u] = *LDS_PTR(bf16x8_t,
                                 q_lds + (c % kQRows) * kQPitch +
                                     16 * q_chunk(half * kKSteps / 2 + u, j));
#pragma unroll
            for (int u = 0; u < kKSteps / 2; ++u)
                s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    k_operand<KV>(rk, half * kKSteps / 2 + u), qb[u], s, 0, 0, 0);
        }
        // Where the loads of the next tile's K go: FP8 tiles are short and
        // latency-bound, so they are issued early, half before the softmax
        // and half after its row maximum; BF16 loads are spread over the P.V
        // MFMAs below, one per two MFMAs (measured fastest of the placements
        // tried: all at once after the scores, spread over the softmax, or
        // alternating with the V loads).
        // The next tile's slots: FP8 needs them here; BF16 resolves them after
        // V(i) is staged, where that wait has already covered their load (a
        // resolve here would wait for V(i) before the scores).
        if constexpr (kMasked) {   // this tile's mask and count, resolved a tile ago
            valid_cur = valid_next;
            bad_total += bad_next;
        }
        int slot_g = 0;
        if constexpr (KV == KvType::kFp8) slot_g = resolve(slot_next);
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
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
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

        wave_lds_fence();   // the previous tile's transpose reads are done
        stage_v<KV, Lay::kVPitch>(rv, vs_lds, lane);
        __builtin_amdgcn_sched_barrier(0);   // V(i) is consumed before V(i+1) lands
        if constexpr (KV == KvType::kBf16) slot_g = resolve(slot_next);
        slot_next = entry_at(tile + (kAhead + 1) * step);
        gather_v<KV, kScalarVAddr>(rv, slot_g, vb, v_ss, lane);
        wave_lds_fence();   // other lanes of this wave wrote the rows read below

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
                                  i16x4_t, vs_lds + tr_row * Lay::kVPitch + 32 * db + 8 * tr_sub)));
            }
#pragma unroll
            for (int u = 0; u < kDimBlocks / 2; ++u) {
                const int db = half * (kDimBlocks / 2) + u;
                o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[u], pb, o[db], 0, 0, 0);
                constexpr int kEvery = kDimBlocks / Gth::kKLoads;
                if (KV == KvType::kBf16 && db % kEvery == kEvery - 1) {
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
            tile_body(tile + b * step, rkb[b], rvb[b]);
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
template <bool kSplit, KvType KV, int kQRows, int kItems = kItemsPerCU, bool kMasked = false>
__global__ __launch_bounds__(64, (AttendLayout<kQRows, kItems>::kWavesPerSimd)) void attend_kernel(
    const AttendParams p) {
    using Lay = AttendLayout<kQRows, kItems>;
    __shared__ __attribute__((aligned(16))) char smem[Lay::kLds];
    if (p.choice != nullptr && ((*p.choice == 1) != (p.choice_value == 1))) return;
    if constexpr (Lay::kPersistent) {
        for (int64_t unit = blockIdx.x; unit < p.units; unit += gridDim.x) {
            wave_lds_fence();   // the previous unit's LDS reads are done
            attend_unit<kSplit, KV, kQRows, kItems, kMasked>(p, unit, smem);
        }
    } else {
        attend_unit<kSplit, KV, kQRows, kItems, kMasked>(p, blockIdx.x, smem);
    }
}

// ---------------------------------------------------------------- merge

// out[t, h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the parts s,
// M = max_s m_s; exactly +0.0 when no part saw a slot.  One wave per (t, h)
// row, 4 dims per lane.  Lane s of each run of 64 parts loads part s's (m, l)
// and computes its weight; the O rows are then read 8 parts at a time, all 8
// loads in flight together, each scaled by its part's weight (a readlane).
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t rows = p.T * p.Hq;
    if (row >= rows) return;
    const int64_t t = row / p.Hq;
    const int h = (int)(row - t * p.Hq);
    const int64_t n = p.n_parts;
    if (p.bad_part != nullptr && h == 0) {
        // The invalid entries of token t's row, reported by its raw-row shares.
        int bad = 0;
        for (int64_t s = lane; s < n; s += 64) bad += p.bad_part[s * p.T + t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) bad += __shfl_xor(bad, off);
        if (lane == 0) p.n_bad[t] = bad;
    }
    float mmax = kNegInf;
    for (int64_t s0 = 0; s0 < n; s0 += 64) {
        const int64_t s = s0 + lane;
        if (s < n) mmax = fmaxf(mmax, p.part_ml[(s * rows + row) * 2]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, off));
    bf16x4_t ob = {(__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
    if (mmax != kNegInf) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        float l_part = 0.0f;
        for (int64_t s0 = 0; s0 < n; s0 += 64) {
            const int64_t s = s0 + lane;
            float w = 0.0f;
            if (s < n) {
                w = __builtin_amdgcn_exp2f(p.part_ml[(s * rows + row) * 2] - mmax);
                l_part += w * p.part_ml[(s * rows + row) * 2 + 1];
            }
            const int cnt = (int)min<int64_t>(64, n - s0);
            for (int u = 0; u < cnt; u += 8) {
                f32x4_t o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[e] = u + e < cnt ? *(const f32x4_t *)(p.part_o + ((s0 + u + e) * rows + row) *
                                                                       kHeadDim + 4 * lane)
                                       : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (u + e < cnt)   // lane u + e holds that part's weight
                        acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u + e)) *
                               o[e];
            }
        }
        float l_tot = l_part;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) l_tot += __shfl_xor(l_tot, off);
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[i] = (__bf16)(acc[i] / l_tot);
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
    if (lane == 0)
        *p.choice = (len > 0.0f && p.lambda_scale * common < p.threshold * len) ? 1 : 0;
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
    const int n = p.count[t];
    const int ntiles = (n + kTileSlots - 1) / kTileSlots;
    const int32_t *list = p.list + t * p.list_stride;
    const char *kb = (const char *)p.k + (int64_t)g * p.k_sh * Gth::kElemBytes;
    const char *vb = (const char *)p.v + (int64_t)g * p.v_sh * Gth::kElemBytes;
    const int64_t k_ss = p.k_ss * Gth::kElemBytes, v_ss = p.v_ss * Gth::kElemBytes;

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

// ---------------------------------------------------------------- indexer

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
constexpr int kScoreSplit = 1024;
constexpr int kIndexRowBytes = kIndexDim * 2;   // 256 B
constexpr int kScoreOutPitch = kScoreTile + 4;  // floats per staged row (16-byte aligned)

// LDS byte offset of 16-byte chunk `chunk` of index-key tile row `r`.  The
// chunk index is XOR-swizzled by a bijection of r & 7 so that the 8 rows read
// by one phase of a 16-byte read hit 8 different bank groups.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int idx_off(int r, int chunk) {
    return r * kIndexRowBytes + ((chunk ^ swz(r)) << 4);
}

__global__ __launch_bounds__(256) void indexer_scores_kernel(const IndexerScoreParams p) {
    // One key tile: the barrier after each tile's scores also orders its reads
    // before the next tile is written.
    __shared__ __attribute__((aligned(16))) char tile[kScoreTile * kIndexRowBytes];
    __shared__ __attribute__((aligned(16))) float out_tile[kScoreTokens * kScoreOutPitch];
    __shared__ int c_end_shared;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c = lane & 15, j = lane >> 4;
    const int64_t t0 = (int64_t)blockIdx.x * kScoreTokens;
    const int c_begin = blockIdx.y * kScoreSplit;

    if (tid == 0) c_end_shared = 0;
    __syncthreads();
    if (tid < kScoreTokens && t0 + tid < p.T) {
        const int64_t lim = ((int64_t)p.positions[t0 + tid] + 1) / kIndexBlock;
        atomicMax(&c_end_shared, (int)min<int64_t>(lim, p.C));
    }
    __syncthreads();
    const int c_end = min(c_end_shared, c_begin + kScoreSplit);
    if (c_begin >= c_end) return;

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

    u32x4_t stage[4];
    load_tile(c_begin, stage);
    for (int c0 = c_begin; c0 < c_end; c0 += kScoreTile) {
        store_tile(tile, stage);
        __syncthreads();   // the key tile is staged; the previous scores are stored
        if (c0 + kScoreTile < c_end) load_tile(c0 + kScoreTile, stage);
#pragma unroll
        for (int ct = 0; ct < kScoreTile / 16; ++ct) {
            bf16x8_t kb[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kb[ks] = *LDS_PTR(bf16x8_t, tile + idx_off(16 * ct + c, 4 * ks + j));
#pragma unroll
            for (int rt = 0; rt < kScoreRowTiles; ++rt) {
                f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rt][ks], kb[ks], d, 0, 0, 0);
                const float score = fmaxf(d[0], 0.f) + fmaxf(d[1], 0.f) + fmaxf(d[2], 0.f) +
                                    fmaxf(d[3], 0.f);
                out_tile[((kScoreTokens / 4) * wave + 4 * rt + j) * kScoreOutPitch + 16 * ct + c] = score;
            }
        }
        __syncthreads();   // the tile's scores are complete
        // kScoreTokens rows of 64 scores: 16 chunks of 4 per row.
#pragma unroll
        for (int u = 0; u < kScoreTokens * (kScoreTile / 4) / 256; ++u) {
            const int idx = tid + 256 * u;
            const int r = idx >> 4, k4 = 4 * (idx & 15);
            const int64_t t_out = t0 + r;
            const int64_t blk = c0 + k4;
            if (t_out < p.T && blk < c_end) {
                const f32x4_t v = *(const f32x4_t *)(out_tile + r * kScoreOutPitch + k4);
                float *dst = p.scores + t_out * p.C + blk;
                if (vec_out && blk + 3 < c_end) {
                    *(f32x4_t *)dst = v;
                } else {
                    for (int e = 0; e < 4 && blk + e < c_end; ++e) dst[e] = v[e];
                }
            }
        }
    }
}

// Order-preserving map of FP32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t score_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
    using Scan = hipcub::BlockScan<int, 256>;
    using Reduce = hipcub::BlockReduce<float, 256>;
    __shared__ float vals[kInLds ? kSelectLdsBlocks : 1];
    __shared__ int hist[256];
    __shared__ int chunk_gt[256], chunk_eq[256];
    __shared__ union {
        typename Scan::TempStorage scan;
        typename Reduce::TempStorage reduce;
    } tmp;
    __shared__ uint32_t sh_prefix;
    __shared__ int sh_need;
    __shared__ float sh_lo, sh_hi;
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
        lo = Reduce(tmp.reduce).Reduce(lo, [](float a, float b) { return fminf(a, b); });
        __syncthreads();
        hi = Reduce(tmp.reduce).Reduce(hi, [](float a, float b) { return fmaxf(a, b); });
        if (tid == 0) {
            sh_lo = lo;
            sh_hi = hi;
        }
        __syncthreads();
        lo = sh_lo;
        hi = sh_hi;
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
        int gt_pre, eq_pre, gt_tot, eq_tot;
        Scan(tmp.scan).ExclusiveSum(my_gt, gt_pre, gt_tot);
        __syncthreads();
        Scan(tmp.scan).ExclusiveSum(my_eq, eq_pre, eq_tot);
        __syncthreads();
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

// Marks, in the first output word, a row that indexer_select_fast_kernel
// left to the exact selection (no output word holds a value below -1).
constexpr int32_t kSelDeferred = INT32_MIN;

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
constexpr int kSelCandSmall = 2048;
constexpr int kSelPerThread = 16;   // scores per thread per pass over the row
// Candidate i is stored at i + i / 16: the output pass, where thread t reads
// candidates kPer t .. kPer t + kPer - 1, then reads different banks.
__device__ __forceinline__ int cand_at(int i) { return i + (i >> 4); }

template <int kCand, int kWavesPerSimd, bool kDefer>
__global__ __launch_bounds__(256, kWavesPerSimd) void indexer_select_fast_kernel(
    const IndexerSelectParams p) {
    static_assert(kCand % 256 == 0 && kCand >= kSelSample, "candidate list");
    // One 16-byte sample load per thread; runs 16 apart or more once n > kCand >= kSelSample.
    static_assert(kSelSample == 4 * 256, "sample runs");
    constexpr int kCandPadded = kCand + kCand / 16;
    using Scan = hipcub::BlockScan<int, 256>;
    __shared__ float cval[kCandPadded];
    __shared__ int cid[kCandPadded];
    __shared__ int hist[256];
    __shared__ typename Scan::TempStorage scan;
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
        for (int e = tid; e < n; e += 256) out[kIndexBlock * e] = e;
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
            int off, total;
            Scan(scan).ExclusiveSum(cnt, off, total);
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
            __syncthreads();   // the scan storage is reused
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
            }
        } else {
            // 3. Exact threshold key tau among the candidates and how many
            // keys equal to tau to keep.
            radix_select(nc, p.budget, [&](int i) { return cval[cand_at(i)]; }, all, hist,
                         &sh_prefix, &sh_need);
            const uint32_t tau = sh_prefix;
            const int need = sh_need;
            // 4. Output in block order.  Thread t owns candidates
            // [kPer t, kPer (t + 1)); a kept candidate's position is the
            // number of keys > tau before it plus the number of kept ties
            // (the first `need` in block order) before it.
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
            int gt_pre, eq_pre, total;
            Scan(scan).ExclusiveSum(gt, gt_pre, total);
            __syncthreads();
            Scan(scan).ExclusiveSum(eq, eq_pre, total);
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int i = kPer * tid + k;
                if (i < nc) {
                    const uint32_t u = score_key(cval[cand_at(i)]);
                    if (u > tau) {
                        out[kIndexBlock * (gt_pre + min(eq_pre, need))] = cid[cand_at(i)];
                        ++gt_pre;
                    } else if (u == tau) {
                        if (eq_pre < need) out[kIndexBlock * (gt_pre + eq_pre)] = cid[cand_at(i)];
                        ++eq_pre;
                    }
                }
            }
        }
    }
    expand_row(p, pos, min(n, p.budget), out, width);
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerScoreParams &p, hipStream_t stream) {
    if (p.T == 0 || p.C == 0) return hipSuccess;
    const int64_t blocks = (p.T + kScoreTokens - 1) / kScoreTokens;
    const int64_t splits = (p.C + kScoreSplit - 1) / kScoreSplit;
    hipLaunchKernelGGL(indexer_scores_kernel, dim3((unsigned)blocks, (unsigned)splits), dim3(256),
                       0, stream, p);
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

// CUs of the current device, queried once per device.
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
template <bool kSplit, KvType KV, int kQRows, int kItems = kItemsPerCU, bool kMasked = false>
void launch_attend_kernel(AttendParams p, int64_t units, hipStream_t stream) {
    using Lay = AttendLayout<kQRows, kItems>;
    p.units = units;
    int64_t grid = units;
    if (Lay::kPersistent) {
        const int64_t full = std::max<int64_t>(
            kXcds, (int64_t)Lay::kItems * device_cus() / kXcds * kXcds);
        grid = std::min(units, full);
    }
    hipLaunchKernelGGL((attend_kernel<kSplit, KV, kQRows, kItems, kMasked>), dim3((unsigned)grid),
                       dim3(64), 0, stream, p);
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
    if (share == nullptr || (kv == KvType::kFp8 && p.G <= 8)) {
        launch_attend_any<false>(p, kv, items, stream);
        return hipGetLastError();
    }
    // The estimate picks one of two launches of the general layout; the other
    // returns at once.  Both compute the same bits.
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
    return hipGetLastError();
}

hipError_t launch_attend_partial(const AttendParams &p, KvType kv, int64_t T,
                                 hipStream_t stream) {
    const int64_t blocks = T * (int64_t)p.Hkv * p.HB * p.splits;
    if (blocks == 0) return hipSuccess;
    if (p.raw_rows) {
        if (kv != KvType::kBf16 || (p.raw == nullptr && p.W_raw > 0)) return hipErrorInvalidValue;
        launch_attend_kernel<true, KvType::kBf16, 16, kItemsPerCU, true>(p, blocks, stream);
        return hipGetLastError();
    }
    launch_attend_any<true>(p, kv, blocks, stream);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeParams &p, hipStream_t stream) {
    const int64_t rows = p.T * p.Hq;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p);
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
