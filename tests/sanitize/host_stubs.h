// Records of the launches the C-ABI layer asked for (see host_stubs.cpp).
#pragma once

#include <vector>

#include "qsa_indexer.h"
#include "qsa_kernels.h"
#include "qsa_measure.h"

namespace stub {

struct Calls {
    std::vector<qsa::CompactParams> compact;
    std::vector<qsa::AttendParams> attend, partial;
    std::vector<qsa::KvType> attend_kv;
    std::vector<int64_t> attend_T;
    std::vector<bool> attend_shared;
    std::vector<qsa::SharingParams> share;
    std::vector<qsa::MergeParams> merge;
    std::vector<qsa::GatherParams> gather;
    std::vector<qsa::IndexerEstimateParams> estimate;
    std::vector<qsa::IndexerScoreParams> scores;
    std::vector<qsa::IndexerSelectParams> select;
    std::vector<qsa::StreamParams> stream;
    std::vector<int64_t> stream_wgs;
    void clear() { *this = Calls(); }
};

extern Calls calls;

}  // namespace stub
