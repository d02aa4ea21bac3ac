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

// Keys of one score workgroup's range (and of one candidate segment).
constexpr int kScoreSplit = 1024;
// Largest budget (blocks) of the fused Top-K path (qsa_indexer_topk), and the
// most key ranges it takes (the select kernel scans one count per thread).
constexpr int kFusedBudgetMax = 512;
constexpr int kFusedMaxRanges = 256;

struct IndexerScoreParams {
    const uint16_t *iq;       // [T, 4, 128]
    int64_t q_st, q_sh;
    const uint16_t *ik;       // [C, 128]
    int64_t k_st;
    int64_t T, C;
    const int32_t *positions; // [T]
    float *scores;            // [T, C]
    // Candidate mode (tau non-null): instead of every score, token t keeps the
    // scores of its eligible blocks whose order-preserving key (see the
    // kernels) is at least tau[t], in block order, as (score, block id)
    // pairs in the part of its row that covers the workgroup's key range
    // (range r = blocks r * kScoreSplit ..): at most half as many pairs as
    // the range has blocks; the count (which may exceed that) goes to
    // counts[t * R + r].
    // The pairs of token t start at scores + t * pair_pitch (pair_pitch even,
    // at least C, so every pair is 8-byte aligned).
    const uint32_t *tau;
    int32_t *counts;
    int64_t R, pair_pitch;
    // Deferred-rows mode (deferred non-null): a workgroup computes its scores
    // only if the first output word of one of its tokens' selection rows
    // holds the deferral mark.
    const int32_t *deferred;
    int64_t deferred_stride;
};

// The sampled threshold estimate of the fused Top-K path: tau[t] = a key that
// about 2 * budget of the token's eligible scores reach (0 for rows of at
// most 2,048 eligible blocks).
struct IndexerEstimateParams {
    const uint16_t *iq;
    int64_t q_st, q_sh;
    const uint16_t *ik;
    int64_t k_st;
    int64_t T, C, L;
    const int32_t *positions;
    int32_t budget;
    uint32_t *tau;            // [T]
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
    // Fused path: per-range candidate counts and the row pitch of the
    // candidate pairs (see IndexerScoreParams).
    const int32_t *counts;
    int64_t R, pair_pitch;
};

hipError_t launch_indexer_scores(const IndexerScoreParams &p, hipStream_t stream);
hipError_t launch_indexer_select(const IndexerSelectParams &p, hipStream_t stream);
// The fused Top-K of qsa_indexer_topk (budget <= kFusedBudgetMax, at most
// kFusedMaxRanges key ranges): the sampled estimate, the scores kept as
// candidates, the exact selection on them, and for rows where the estimate
// missed (too few or too many candidates) the full scores and the exact
// selection on those.
hipError_t launch_indexer_topk_fused(const IndexerEstimateParams &e, const IndexerScoreParams &s,
                                     const IndexerSelectParams &p, hipStream_t stream);

}  // namespace qsa
