// qsa_sparse_prefill_noalloc: the sparse prefill for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its workspace is a fixed array in device
// memory that the library's code object holds on every GPU it runs on, until
// the process ends.  Every call on one GPU uses that GPU's copy, so calls that
// overlap on one GPU (different streams, or threads) race on it.
//
// The array's name in host code is a host-side stand-in, not its device
// address: the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to the kernels.

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "qsa.h"
#include "qsa_errors.h"

namespace {

// The prefill's workspace (qsa_workspace_bytes(T, W) bytes): at most this.
// 64 MiB holds the long prefill of 7,810 tokens x 2,051 entries (62.1 MiB).
constexpr size_t kScratchBytes = size_t(64) << 20;

__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];

// The current device's copy of `scratch`, looked up on the first call on that
// device; NULL (with *err set) if the lookup fails.
void *scratch_on_current_device(hipError_t *err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" {

size_t qsa_noalloc_scratch_bytes(void) { return kScratchBytes; }

qsa_status qsa_sparse_prefill_noalloc(const qsa_bf16_view *q, const qsa_bf16_view *k_cache,
                                      const qsa_bf16_view *v_cache, const qsa_i32_view *slot_idx,
                                      float scale, qsa_bf16_view *out, void *stream) {
    if (!slot_idx) {
        // The refusal of the allocating entry point, message included.
        return qsa_sparse_prefill(q, k_cache, v_cache, slot_idx, scale, out, nullptr, 0, stream);
    }
    const int64_t T = slot_idx->size[0], W = slot_idx->size[1];
    const size_t need = qsa_workspace_bytes(T, W);
    if (need > kScratchBytes)
        return (qsa_status)qsa::set_error(QSA_ERR_UNSUPPORTED,
                              "qsa_sparse_prefill_noalloc: %lld tokens x %lld entries need %zu "
                              "bytes of workspace; its fixed scratch holds %zu (use "
                              "qsa_sparse_prefill with a workspace, or split the tokens)",
                              (long long)T, (long long)W, need, kScratchBytes);
    hipError_t e = hipSuccess;
    void *ws = scratch_on_current_device(&e);
    if (ws == nullptr)
        return (qsa_status)qsa::set_error(QSA_ERR_HIP, "scratch address lookup: %s", hipGetErrorString(e));
    // Nothing in the workspace has to start at zero: the compaction writes
    // every word the attention reads.
    return qsa_sparse_prefill(q, k_cache, v_cache, slot_idx, scale, out, ws, kScratchBytes,
                              stream);
}

}  // extern "C"
