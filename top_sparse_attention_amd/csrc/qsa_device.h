// Device-side helpers shared by the HIP kernels of libqsa (gfx950).  Not
// part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

constexpr float kNegInf = -__builtin_huge_valf();

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

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace
}  // namespace qsa
