// Internal launchers of the QSA indexer and Top-K selection, shared by the
// C-ABI layer and the HIP kernels.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// QSA indexer: 4 query heads sharing one key head, head dim 128, one key per
// block of 4 positions.
constexpr int kIndexHeads = 4;
constexpr int kIndexDim = 128;
constexpr int kIndexBlock = 4;
// Blocks per row that the select kernel keeps in LDS (larger rows are read
// from global memory on every pass).
constexpr int kSelectLdsBlocks = 16384;

struct IndexerScoreParams {
    const uint16_t *iq;       // [T, 4, 128]
    int64_t q_st, q_sh;
    const uint16_t *ik;       // [C, 128]
    int64_t k_st;
    int64_t T, C;
    const int32_t *positions; // [T]
    float *scores;            // [T, C]
};

struct IndexerSelectParams {
    const float *scores;      // [T, C]
    int64_t T, C;
    const int32_t *positions; // [T]; a row whose position is outside [0, L) is all -1
    const int32_t *slot_of_pos; // [L]
    int64_t L;
    int32_t budget;
    int32_t *out;             // [T, out_stride], width 4 * budget + 3
    int64_t out_stride;
};

hipError_t launch_indexer_scores(const IndexerScoreParams &p, hipStream_t stream);
hipError_t launch_indexer_select(const IndexerSelectParams &p, hipStream_t stream);

}  // namespace qsa
