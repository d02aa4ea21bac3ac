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
// Two passes:
//  1. compact_kernel: per token row, a stable filter of the selection list
//     (keeps entries in [0, S) in input order, counts the rest as invalid),
//     padded with -1 to a multiple of the tile size.
//  2. attend_kernel: one work item = (token t, KV head g, block of up to 16
//     query heads of that group).  kWavesPerItem waves split the item's
//     32-slot tiles round-robin; each wave gathers its tile's K and V rows
//     (512 B each, 16-byte coalesced loads, double-buffered through
//     registers), stages them in LDS, computes the 32x16 score tile with
//     bf16 MFMA (K rows x query heads), runs an online softmax in FP32,
//     and accumulates P.V with bf16 MFMA reading V through LDS transpose
//     loads.  The waves' partial (max, sum, O) are merged through LDS at
//     the end and the row is written in BF16.
//
// MFMA orientation: scores are computed transposed, S^T = K_tile . Q^T, so
// that one lane owns one query head (column) of the MFMA output: the row
// maximum needs only two cross-lane steps and the O rescale is one scalar per
// lane.  The output O^T = V^T . P^T uses the same lane-to-head map.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa_kernels.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))
#define GLOBAL_PTR(T, p) ((const __attribute__((address_space(1))) T *)(p))

constexpr int kRowBytes = kHeadDim * 2;          // one K or V row: 512 B
constexpr int kChunksPerRow = kRowBytes / 16;    // 32 sixteen-byte chunks
constexpr int kTileBytes = kTileSlots * kRowBytes;  // 16 KiB of K (or V)
constexpr int kWaveLds = 2 * kTileBytes;         // K tile + V tile per wave
constexpr int kThreads = 64 * kWavesPerItem;
constexpr int kLoadsPerTile = kTileBytes / (64 * 16);  // 16 dwordx4 per lane
constexpr float kNegInf = -__builtin_huge_valf();
// A new running maximum is adopted only when it exceeds the current one by
// more than this (log2 units); otherwise probabilities may reach 2^8, which
// FP32 sums and BF16 probabilities hold exactly as well.  This skips most
// rescales of the O accumulators.
constexpr float kRescaleSlack = 8.0f;

// A row of zeros: masked tile rows and absent query heads load from here, so
// every load is unconditional and no select waits on loaded data.
__device__ __attribute__((aligned(16))) uint16_t kZeroRow[kHeadDim] = {};

// 16-byte load through the global address space (all operands of the
// gathers, including kZeroRow, are global memory; a generic pointer would
// turn the loads into flat loads).
template <typename V>
__device__ __forceinline__ V ldg16(const void *p) {
    return *GLOBAL_PTR(V, p);
}

// LDS byte offset of 16-byte chunk `chunk` of tile row `r`.  The chunk index
// is XOR-swizzled by a bijection of r & 7 so that (a) the 8 rows read by one
// ds_read_b128 phase of the score MFMA hit 8 different bank groups, and (b)
// the 4 rows read by one 16-lane group of the V transpose loads hit 4
// different 32-byte bank windows.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
__device__ __forceinline__ int lds_off(int r, int chunk) {
    return r * kRowBytes + ((chunk ^ swz(r)) << 4);
}

// ---------------------------------------------------------------- compaction

__global__ __launch_bounds__(256) void compact_kernel(const CompactParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= p.T) return;
    const int32_t *src = p.slot_idx + t * p.stride_t;
    int32_t *dst = p.list + t * p.row_stride;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    int n = 0, bad = 0;
    for (int64_t base = 0; base < p.W; base += 256) {
        int32_t e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + u * 64 + lane;
            e[u] = i < p.W ? src[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool ok = e[u] >= 0 && (int64_t)e[u] < p.S;
            const uint64_t keep = __ballot(ok);
            if (ok) dst[n + __popcll(keep & below)] = e[u];
            n += __popcll(keep);
            bad += __popcll(__ballot(!ok && e[u] != -1));
        }
    }
    const int padded = (n + kTileSlots - 1) & ~(kTileSlots - 1);
    for (int i = n + lane; i < padded; i += 64) dst[i] = -1;
    if (lane == 0) {
        p.count[t] = n;
        p.n_bad[t] = bad;
    }
}

// ---------------------------------------------------------------- gathers

// Issue the 2 x 16 dwordx4 loads of one tile.  `slot` holds, in lane r (and
// r + 32), the slot of tile row r (-1: none).  Load q covers rows 2q (lanes
// 0-31) and 2q+1 (lanes 32-63), one 16-byte chunk per lane, so each row is
// one fully coalesced 512-byte read.
__device__ __forceinline__ void gather_tile(u32x4_t (&rk)[kLoadsPerTile],
                                            u32x4_t (&rv)[kLoadsPerTile], int slot,
                                            const uint16_t *kb, int64_t k_ss,
                                            const uint16_t *vb, int64_t v_ss, int lane) {
    const int ch8 = (lane & 31) * 8;
    const bool upper = lane >= 32;
#pragma unroll
    for (int q = 0; q < kLoadsPerTile; ++q) {
        const int s_lo = __builtin_amdgcn_readlane(slot, 2 * q);
        const int s_hi = __builtin_amdgcn_readlane(slot, 2 * q + 1);
        const int s = upper ? s_hi : s_lo;
        const uint16_t *kp = s >= 0 ? kb + (int64_t)s * k_ss + ch8 : kZeroRow + ch8;
        const uint16_t *vp = s >= 0 ? vb + (int64_t)s * v_ss + ch8 : kZeroRow + ch8;
        rk[q] = ldg16<u32x4_t>(kp);
        rv[q] = ldg16<u32x4_t>(vp);
    }
}

__device__ __forceinline__ void stage_tile(const u32x4_t (&rk)[kLoadsPerTile],
                                           const u32x4_t (&rv)[kLoadsPerTile],
                                           char *ks, char *vs, int lane) {
    const int ch = lane & 31;
    const int half = lane >> 5;
#pragma unroll
    for (int q = 0; q < kLoadsPerTile; ++q) {
        const int off = lds_off(2 * q + half, ch);
        *LDS_PTR(u32x4_t, ks + off) = rk[q];
        *LDS_PTR(u32x4_t, vs + off) = rv[q];
    }
}

// ---------------------------------------------------------------- attention

__global__ __launch_bounds__(kThreads, 1) void attend_kernel(const AttendParams p) {
    __shared__ __attribute__((aligned(16))) char smem[kWavesPerItem * kWaveLds];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;   // MFMA column: query head within the block / A-operand row
    const int j = lane >> 4;   // MFMA lane group

    const int64_t item = blockIdx.x;
    const int64_t per_t = (int64_t)p.Hkv * p.HB;
    const int64_t t = item / per_t;
    const int rem = (int)(item - t * per_t);
    const int g = rem / p.HB;
    const int hb = rem - g * p.HB;
    const int h0 = g * p.G + hb * 16;
    const int nh = min(16, p.G - hb * 16);
    const int n = p.count[t];

    uint16_t *out_t = p.out + t * p.o_st + (int64_t)h0 * p.o_sh;
    if (n == 0) {
        // Nothing selected: the output row is exactly +0.0.
        for (int idx = threadIdx.x; idx < nh * kChunksPerRow; idx += kThreads) {
            const int hh = idx / kChunksPerRow, ch = idx % kChunksPerRow;
            *(u32x4_t *)(out_t + hh * p.o_sh + ch * 8) = u32x4_t{0, 0, 0, 0};
        }
        return;
    }

    // Query heads as the B operand of S^T = K . Q^T: lane (c, j) holds head c,
    // dims 32 ks + 8 j .. +8 for k-step ks.
    bf16x8_t qb[8];
    {
        const uint16_t *qrow = c < nh ? p.q + t * p.q_st + (int64_t)(h0 + c) * p.q_sh : kZeroRow;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qb[ks] = ldg16<bf16x8_t>(qrow + 32 * ks + 8 * j);
    }

    const int ntiles = (n + kTileSlots - 1) / kTileSlots;
    const int32_t *list = p.list + t * p.list_stride;
    const uint16_t *kb = p.k + (int64_t)g * p.k_sh;
    const uint16_t *vb = p.v + (int64_t)g * p.v_sh;
    char *ks_lds = smem + wave * kWaveLds;
    char *vs_lds = ks_lds + kTileBytes;

    float m = kNegInf;   // running max (log2 domain) for head c
    float lsum = 0.0f;   // this lane's share of the softmax denominator
    f32x4_t o[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t rk[kLoadsPerTile], rv[kLoadsPerTile];
    int tile = wave;
    int slot_next = -1;
    if (tile < ntiles) {
        const int slot_cur = list[tile * kTileSlots + (lane & 31)];
        if (tile + kWavesPerItem < ntiles)
            slot_next = list[(tile + kWavesPerItem) * kTileSlots + (lane & 31)];
        gather_tile(rk, rv, slot_cur, kb, p.k_ss, vb, p.v_ss, lane);
    }

    for (; tile < ntiles; tile += kWavesPerItem) {
        // The previous tile's LDS reads must be done before it is overwritten.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        stage_tile(rk, rv, ks_lds, vs_lds, lane);
        const int nt = tile + kWavesPerItem;
        if (nt < ntiles) {
            gather_tile(rk, rv, slot_next, kb, p.k_ss, vb, p.v_ss, lane);
            slot_next = nt + kWavesPerItem < ntiles
                            ? list[(nt + kWavesPerItem) * kTileSlots + (lane & 31)]
                            : -1;
        }
        // Other lanes of this wave wrote the rows read below.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // S^T for the two 16-slot blocks: s0[i] / s1[i] = score of tile slot
        // 4j+i / 16+4j+i against head c.
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        bf16x8_t ka[2][8];
#pragma unroll
        for (int kstep = 0; kstep < 8; ++kstep) {
            ka[0][kstep] = *LDS_PTR(bf16x8_t, ks_lds + lds_off(c, 4 * kstep + j));
            ka[1][kstep] = *LDS_PTR(bf16x8_t, ks_lds + lds_off(16 + c, 4 * kstep + j));
        }
#pragma unroll
        for (int kstep = 0; kstep < 8; ++kstep) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0][kstep], qb[kstep], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1][kstep], qb[kstep], s1, 0, 0, 0);
        }

        // Online softmax in the log2 domain; slots at or past n are masked.
        const int first = tile * kTileSlots + 4 * j;
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = first + i < n ? s0[i] * p.scale_log2e : kNegInf;
            x[4 + i] = first + 16 + i < n ? s1[i] * p.scale_log2e : kNegInf;
        }
        float mt = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mt = fmaxf(mt, x[i]);
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const bool raise = mt > m + kRescaleSlack;
        const float m_new = raise ? mt : m;
        if (__ballot(raise)) {
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < 16; ++db) o[db] *= alpha;
        }
        m = m_new;
        bf16x8_t pb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const __bf16 pr = (__bf16)__builtin_amdgcn_exp2f(x[i] - m);
            pb[i] = pr;
            lsum += (float)pr;
        }

        // O^T += V^T . P^T.  The k index (slot) runs over tile slots 4j..4j+3
        // then 16+4j..16+4j+3 for lane group j, matching pb.  Each half comes
        // from one ds_read_b64_tr_b16: lane i of a 16-lane group addresses
        // row R0 + i/4, dims 16 db + 4 (i%4); lane c then receives
        // V[R0 + e][16 db + c] for e = 0..3.
        const int tr_row0 = 4 * j + (c >> 2);
        const int tr_sub = (c & 3);
        bf16x8_t va[16];
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            const int chunk = 2 * db + (tr_sub >> 1);
            const int byte_in = 8 * (tr_sub & 1);
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                LDS_PTR(i16x4_t, vs_lds + lds_off(tr_row0, chunk) + byte_in));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                LDS_PTR(i16x4_t, vs_lds + lds_off(16 + tr_row0, chunk) + byte_in));
            va[db] = __builtin_bit_cast(
                bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int db = 0; db < 16; ++db)
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pb, o[db], 0, 0, 0);
    }

    // Whole-head denominator of this wave: add the four lane groups.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    // Merge the waves' partial states through LDS (reusing the tile area).
    __syncthreads();
    f32x4_t *part_o = (f32x4_t *)smem;                        // [wave][db][lane]
    float *part_m = (float *)(smem + kWavesPerItem * 16 * 64 * 16);  // [wave][16]
    float *part_l = part_m + kWavesPerItem * 16;                      // [wave][16]
#pragma unroll
    for (int db = 0; db < 16; ++db) part_o[(wave * 16 + db) * 64 + lane] = o[db];
    if (j == 0) {
        part_m[wave * 16 + c] = m;
        part_l[wave * 16 + c] = lsum;
    }
    __syncthreads();

    float mw[kWavesPerItem], fw[kWavesPerItem];
    float mmax = kNegInf;
#pragma unroll
    for (int w = 0; w < kWavesPerItem; ++w) {
        mw[w] = part_m[w * 16 + c];
        mmax = fmaxf(mmax, mw[w]);
    }
    float l_tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerItem; ++w) {
        fw[w] = __builtin_amdgcn_exp2f(mw[w] - mmax);   // 0 for waves without tiles
        l_tot += fw[w] * part_l[w * 16 + c];
    }
    constexpr int kDbPerWave = 16 / kWavesPerItem;
    if (c < nh) {
        uint16_t *orow = out_t + (int64_t)c * p.o_sh;
#pragma unroll
        for (int d = 0; d < kDbPerWave; ++d) {
            const int db = wave * kDbPerWave + d;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kWavesPerItem; ++w) acc += fw[w] * part_o[(w * 16 + db) * 64 + lane];
            bf16x4_t ob;
#pragma unroll
            for (int i = 0; i < 4; ++i) ob[i] = (__bf16)(acc[i] / l_tot);
            *(u32x2_t *)(orow + 16 * db + 4 * j) = __builtin_bit_cast(u32x2_t, ob);
        }
    }
}

// ---------------------------------------------------------------- gather ceiling

// Reads the same rows with the same tiles, waves and load pattern as
// attend_kernel, folds them with XOR and writes one word per (t, g).
__global__ __launch_bounds__(kThreads, 1) void ceiling_kernel(const CeilingParams p) {
    __shared__ uint32_t fold[kWavesPerItem];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t item = blockIdx.x;
    const int64_t t = item / p.Hkv;
    const int g = (int)(item - t * p.Hkv);
    const int n = p.count[t];
    const int ntiles = (n + kTileSlots - 1) / kTileSlots;
    const int32_t *list = p.list + t * p.list_stride;
    const uint16_t *kb = p.k + (int64_t)g * p.k_sh;
    const uint16_t *vb = p.v + (int64_t)g * p.v_sh;

    u32x4_t acc = {0, 0, 0, 0};
    u32x4_t rk[kLoadsPerTile], rv[kLoadsPerTile];
    int tile = wave;
    int slot_next = -1;
    if (tile < ntiles) {
        const int slot_cur = list[tile * kTileSlots + (lane & 31)];
        if (tile + kWavesPerItem < ntiles)
            slot_next = list[(tile + kWavesPerItem) * kTileSlots + (lane & 31)];
        gather_tile(rk, rv, slot_cur, kb, p.k_ss, vb, p.v_ss, lane);
    }
    for (; tile < ntiles; tile += kWavesPerItem) {
#pragma unroll
        for (int q = 0; q < kLoadsPerTile; ++q) acc ^= rk[q] ^ rv[q];
        const int nt = tile + kWavesPerItem;
        if (nt < ntiles) {
            gather_tile(rk, rv, slot_next, kb, p.k_ss, vb, p.v_ss, lane);
            slot_next = nt + kWavesPerItem < ntiles
                            ? list[(nt + kWavesPerItem) * kTileSlots + (lane & 31)]
                            : -1;
        }
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
    if (lane == 0) fold[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
        for (int w = 0; w < kWavesPerItem; ++w) y ^= fold[w];
        p.sink[item] = y;
    }
}

}  // namespace

hipError_t launch_compact(const CompactParams &p, hipStream_t stream) {
    if (p.T == 0) return hipSuccess;
    const int64_t blocks = (p.T + 3) / 4;
    hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_attend(const AttendParams &p, int64_t T, hipStream_t stream) {
    const int64_t items = T * (int64_t)p.Hkv * p.HB;
    if (items == 0) return hipSuccess;
    hipLaunchKernelGGL(attend_kernel, dim3((unsigned)items), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_ceiling(const CeilingParams &p, int64_t T, hipStream_t stream) {
    const int64_t items = T * (int64_t)p.Hkv;
    if (items == 0) return hipSuccess;
    hipLaunchKernelGGL(ceiling_kernel, dim3((unsigned)items), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace qsa
