// Internal launchers shared by the C-ABI layer and the HIP kernels.
// Not part of the public interface (that is include/qsa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Head dim the kernels are written for (the only one the method uses).
constexpr int kHeadDim = 256;
// Slots per gather tile, and the granularity the compacted lists are padded to.
constexpr int kTileSlots = 32;
// Waves that share one (token, KV head, head block) work item.
constexpr int kWavesPerItem = 4;

struct CompactParams {
    const int32_t *slot_idx;
    int64_t stride_t;
    int64_t T, W, S;
    int32_t *list;
    int64_t row_stride;
    int32_t *count;
    int32_t *n_bad;
};

struct AttendParams {
    const uint16_t *q;
    int64_t q_st, q_sh;
    const uint16_t *k;
    int64_t k_ss, k_sh;
    const uint16_t *v;
    int64_t v_ss, v_sh;
    const int32_t *list;
    int64_t list_stride;
    const int32_t *count;
    uint16_t *out;
    int64_t o_st, o_sh;
    int32_t Hkv;
    int32_t G;           // query heads per KV head
    int32_t HB;          // 16-head blocks per KV head: ceil(G / 16)
    float scale_log2e;   // scale * log2(e)
};

struct CeilingParams {
    const uint16_t *k;
    int64_t k_ss, k_sh;
    const uint16_t *v;
    int64_t v_ss, v_sh;
    const int32_t *list;
    int64_t list_stride;
    const int32_t *count;
    uint32_t *sink;
    int32_t Hkv;
};

hipError_t launch_compact(const CompactParams &p, hipStream_t stream);
hipError_t launch_attend(const AttendParams &p, int64_t T, hipStream_t stream);
hipError_t launch_ceiling(const CeilingParams &p, int64_t T, hipStream_t stream);

}  // namespace qsa
