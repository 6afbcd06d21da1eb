// gdn2_peak.hip -- measured fp16 MFMA rates on the device, as context for the
// fraction of the published dense peak that the forward reaches.  Not part
// of the gdn2 C interface: bench.py loads it from libgdn2_peak.so.
//
// kind 0: v_mfma_f32_32x32x16_f16 (32768 flop), 4 independent chains per wave;
// kind 1: v_mfma_f32_16x16x32_f16 (16384 flop), 8 chains per wave -- the
//         instruction the forward's contractions use.
// Every wave runs `iters` rounds over its chains; one float per workgroup is
// written so that the products are kept.
#include <hip/hip_runtime.h>
#include <cstdint>

typedef _Float16 halfx8_p __attribute__((ext_vector_type(8)));
typedef float floatx4_p __attribute__((ext_vector_type(4)));
typedef float floatx16_p __attribute__((ext_vector_type(16)));

template <int KIND>
__global__ __launch_bounds__(256) void peak_mfma_kernel(float* out, int iters) {
    halfx8_p a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)((threadIdx.x + i) & 7) * (_Float16)0.125f;
        b[i] = (_Float16)((threadIdx.x * 3 + i) & 7) * (_Float16)0.0625f;
    }
    float s = 0.f;
    if constexpr (KIND == 0) {
        floatx16_p acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][15];
    } else {
        floatx4_p acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = floatx4_p{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][3];
    }
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

// Enqueues `groups` workgroups of 256 threads on `stream`; out holds `groups`
// floats (device).  Returns 0, or -1 for bad arguments, -4 if the launch
// failed.  Flop per call: groups * 4 * iters * 131072 (either kind).
extern "C" int gdn2_peak_mfma(int32_t kind, float* out, int32_t groups, int32_t iters,
                              void* stream) {
    if (!out || groups < 1 || iters < 1 || kind < 0 || kind > 1) return -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind == 0)
        hipLaunchKernelGGL(peak_mfma_kernel<0>, dim3((unsigned)groups), dim3(256), 0, s, out, iters);
    else
        hipLaunchKernelGGL(peak_mfma_kernel<1>, dim3((unsigned)groups), dim3(256), 0, s, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
