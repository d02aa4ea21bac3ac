// Stand-ins for the kernel launchers of libqsa, for a host-only build of the
// C-ABI layer (qsa_api.cpp) under AddressSanitizer and UBSan: each records
// the parameters it was given and launches nothing, so every host-side path
// of the library (argument checks, workspace layouts, the choice of lists,
// layouts and splits) runs without a GPU.
#include "host_stubs.h"

namespace stub {
Calls calls;
}

namespace qsa {

hipError_t launch_compact(const CompactParams &p, hipStream_t) {
    stub::calls.compact.push_back(p);
    return hipSuccess;
}

hipError_t launch_attend(const AttendParams &p, KvType kv, int64_t T, hipStream_t,
                         const SharingParams *share) {
    stub::calls.attend.push_back(p);
    stub::calls.attend_kv.push_back(kv);
    stub::calls.attend_T.push_back(T);
    stub::calls.attend_shared.push_back(share != nullptr);
    if (share) stub::calls.share.push_back(*share);
    return hipSuccess;
}

hipError_t launch_attend_partial(const AttendParams &p, KvType kv, int64_t T, hipStream_t) {
    stub::calls.partial.push_back(p);
    stub::calls.attend_kv.push_back(kv);
    stub::calls.attend_T.push_back(T);
    return hipSuccess;
}

hipError_t launch_merge(const MergeParams &p, hipStream_t) {
    stub::calls.merge.push_back(p);
    return hipSuccess;
}

hipError_t launch_gather_only(const GatherParams &p, KvType, int64_t, hipStream_t) {
    stub::calls.gather.push_back(p);
    return hipSuccess;
}

hipError_t launch_indexer_scores(const IndexerScoreParams &p, hipStream_t) {
    stub::calls.scores.push_back(p);
    return hipSuccess;
}

hipError_t launch_indexer_select(const IndexerSelectParams &p, hipStream_t) {
    stub::calls.select.push_back(p);
    return hipSuccess;
}

hipError_t launch_indexer_topk_fused(const IndexerEstimateParams &e, const IndexerScoreParams &s,
                                     const IndexerSelectParams &p, hipStream_t) {
    stub::calls.estimate.push_back(e);
    stub::calls.scores.push_back(s);
    stub::calls.select.push_back(p);
    return hipSuccess;
}

hipError_t launch_stream_read(const StreamParams &p, int64_t workgroups, hipStream_t) {
    stub::calls.stream.push_back(p);
    stub::calls.stream_wgs.push_back(workgroups);
    return hipSuccess;
}

}  // namespace qsa
