// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Number of XCDs on MI355X: consecutive workgroup ids are dealt round-robin
// to them, and each XCD has its own L2.
constexpr int kNumXcd = 8;

// Map a hardware workgroup id onto a logical work index so that logical
// indices that are close together (same head, neighbouring query tiles) land
// on the same XCD and share its L2.  `grid` must be a multiple of kNumXcd;
// returns an index in [0, grid).
__device__ __forceinline__ int xcd_swizzle(int bid, int grid) {
    const int per = grid / kNumXcd;
    return (bid % kNumXcd) * per + bid / kNumXcd;
}

__device__ __forceinline__ u32x4 ldg128(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void stg128(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 f = {a, b};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// Value held by lane (lane ^ 32) of the wavefront.
__device__ __forceinline__ float xor32(float x) {
    return __shfl_xor(x, 32, 64);
}

}  // namespace mattn
