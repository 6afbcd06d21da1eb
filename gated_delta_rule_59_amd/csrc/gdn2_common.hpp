// gdn2_common.hpp -- device helpers shared by the gfx950 kernels of this
// library: storage-type conversion, vector types and the MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// bf16 is carried as its raw 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32): round to
// nearest even, NaN stays NaN (quiet).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    floatx2_t f;
    f[0] = lo;
    f[1] = hi;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// ---- loads of 8 consecutive storage elements, widened to fp32 ----------------
__device__ __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
    const u16x8 v = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = bf16_to_f32(v[i]);
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ float load1(const bf16_t* p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ float load1(const float* p) { return *p; }

__device__ __forceinline__ void store1(bf16_t* p, float x) {
    p->bits = static_cast<uint16_t>(f32x2_to_bf16x2(x, 0.f));
}
__device__ __forceinline__ void store1(float* p, float x) { *p = x; }

// Stores 4 consecutive outputs.
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
    uint2 v;
    v.x = f32x2_to_bf16x2(a, b);
    v.y = f32x2_to_bf16x2(c, d);
    *reinterpret_cast<uint2*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// ---- MFMA wrappers (CDNA4, wave64) -------------------------------------------
// Lane l of a 16x16 tile instruction: A row / B column = l & 15, and the lane
// group g = l >> 4 carries a slice of the contraction index.  The output
// holds D[4g + j][l & 15] in element j.  The contraction index may be permuted
// freely as long as the A and B fragments use the same permutation.
__device__ __forceinline__ floatx4 mma16(halfx8 a, halfx8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16(halfx4 a, halfx4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- sums across lanes by lane swaps (gfx950 v_permlane32/16_swap) ----
// lanes 0..31: a(own) + a(lane + 32); lanes 32..63: b(lane - 32) + b(own)
__device__ __forceinline__ float swap32_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// 16-lane rows 0, 2: a(own) + a(lane + 16); rows 1, 3: b(lane - 16) + b(own)
__device__ __forceinline__ float swap16_sum(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x summed over the four lanes l & 15 + 16 g (g = 0..3), in each of them
__device__ __forceinline__ float sum_over_rows16(float x) {
    const float y = swap16_sum(x, x);
    return swap32_sum(y, y);
}

// Chunk slots of the backward's per-chunk buffers (checkpoints of the state
// and the chunk intermediates), 64-token chunks: sequence n owns slots
// ckpt_slot0(n) .. ckpt_slot0(n) + ceil(L_n / 64); the last one holds the
// final state.  Dense batches (cu == null): L_n = T.
__device__ __forceinline__ int64_t ckpt_slot0(const int32_t* cu, int T, int n) {
    if (!cu) return (int64_t)n * ((T + 63) / 64 + 1);
    int64_t s = 0;
    for (int m = 0; m < n; ++m) s += ((int64_t)cu[m + 1] - cu[m] + 63) / 64 + 1;
    return s;
}

__device__ __forceinline__ floatx4 zero4() {
    floatx4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

}  // namespace gdn2
