// Internal launcher of the streaming-read measurement kernel.  Not part of
// the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Streaming read (measurement only): `workgroups` workgroups each read
// chunks_per_wg 16-byte chunks of a footprint of footprint_chunks chunks.
struct StreamParams {
    const void *buf;
    int64_t footprint_chunks;
    int64_t chunks_per_wg;   // <= footprint_chunks
    uint32_t *sink;          // [workgroups]
};

hipError_t launch_stream_read(const StreamParams &p, int64_t workgroups, hipStream_t stream);

}  // namespace qsa
