// Shared device-side helpers of libbsa (gfx950 only). Internal header: not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// MI355X: 8 XCDs, each with its own L2. Workgroups are dispatched to XCDs round-robin
// (workgroup w runs on XCD w % 8). This maps the hardware order to a logical order in
// which each XCD receives one contiguous range of logical work items, so neighbouring
// items (same head, adjacent query blocks, overlapping key blocks) share an L2.
constexpr int kNumXcd = 8;

__device__ __forceinline__ int xcd_remap(int w, int total) {
    int xcd = w % kNumXcd, slot = w / kNumXcd;
    int base = total / kNumXcd, rem = total % kNumXcd;
    int start = xcd * base + (xcd < rem ? xcd : rem);
    return start + slot;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// Round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// A 32-bit key whose unsigned order is the order of the float (-0 folded into +0).
__device__ __forceinline__ uint32_t ordered_key(float s) {
    uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace bsa
