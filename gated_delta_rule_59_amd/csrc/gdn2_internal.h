// gdn2_internal.h -- launchers shared between the C-ABI translation unit and
// the kernel translation units of this library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn2 {

enum { DT_F32 = 0, DT_BF16 = 1 };
// Gate shapes (values of gdn2_gates): per channel, or one value per (token,
// head) broadcast over the channels -- b and w for GATES_KDA, alpha, b and w
// for GATES_GDN.
enum { GATES_FULL = 0, GATES_KDA = 1, GATES_GDN = 2 };

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* alpha,
                         const void* b, const void* w, int in_dtype, float* S, void* o,
                         int out_dtype, int N, int H, int dk, int dv, int gates,
                         hipStream_t stream);

// Token-serial forward (fp32 inputs and output); the chunked kernels' fp32
// tiles do not fit in LDS at dk = 128.  No workspace.
hipError_t launch_fwd_serial(const float* q, const float* k, const float* v, const float* alpha,
                             const float* b, const float* w, const float* S0, float* o,
                             float* S_T, const int32_t* cu_seqlens, int N, int T, int H, int dk,
                             int dv, int gates, hipStream_t stream);

// Forward launch plan; fields are filled by plan_fwd and consumed by launch_fwd.
struct FwdPlan {
    int nslab;            // value slabs per (sequence, head)
    int nslab_m;          // slabs of the dk x dk transition part (summary pass)
    int nseg;             // segments per sequence (1 = no split)
    int seg_chunks;       // chunks per segment
    size_t maps_off;      // workspace offset of the segment maps [pair][seg][dk][dv + dk]
    size_t starts_off;    // workspace offset of the segment start states [pair][seg][dk][dv]
    bool order;           // packed batch: sequence order by length at order_off (int32[num_seqs])
    size_t order_off;
    size_t workspace;     // bytes of device workspace needed
};

FwdPlan plan_fwd(int B, int T, int H, int dk, int dv, int num_seqs, int in_dtype);

hipError_t launch_fwd(const FwdPlan& plan, const void* q, const void* k, const void* v,
                      const void* alpha, const void* b, const void* w, int in_dtype,
                      const float* S0, void* o, int out_dtype, float* S_T,
                      const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int dk,
                      int dv, int gates, void* workspace, hipStream_t stream);

}  // namespace gdn2
