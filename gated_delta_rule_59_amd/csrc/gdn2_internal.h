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

// erase_rows: the erase gate b gates the erased rows instead of the key that
// reads the prediction (the other reading of the pages).
hipError_t launch_decode(const void* q, const void* k, const void* v, const void* alpha,
                         const void* b, const void* w, int in_dtype, float* S, void* o,
                         int out_dtype, int N, int H, int dk, int dv, int gates,
                         hipStream_t stream, bool erase_rows = false);

// Token-serial forward: fp32 inputs at dk = 128 (the chunked kernels' fp32
// tiles do not fit in LDS), and every forward of the erase-on-rows reading.
// With ckpt (fp32 in, fp32 out), no output: the backward's checkpoints
// instead.  With nseg > 1, one pass over segments of seg_chunks chunks:
// summary != 0 writes the segments' state maps to maps, else each segment
// runs from starts (see fwd_serial_kernel).
hipError_t launch_fwd_serial(const void* q, const void* k, const void* v, const void* alpha,
                             const void* b, const void* w, int in_dtype, const float* S0,
                             void* o, int out_dtype, float* S_T, const int32_t* cu_seqlens,
                             int N, int T, int H, int dk, int dv, int gates, bool erase_rows,
                             hipStream_t stream, float* ckpt = nullptr, int nseg = 1,
                             int seg_chunks = 0, int summary = 0, float* maps = nullptr,
                             const float* starts = nullptr);

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

// The token-serial forward under a plan (segmented when plan.nseg > 1:
// summary pass, combine pass, forward pass, with the maps and starts in the
// workspace).
hipError_t launch_fwd_serial_plan(const FwdPlan& plan, const void* q, const void* k,
                                  const void* v, const void* alpha, const void* b, const void* w,
                                  int in_dtype, const float* S0, void* o, int out_dtype,
                                  float* S_T, const int32_t* cu_seqlens, int N, int T, int H,
                                  int dk, int dv, int gates, bool erase_rows, void* workspace,
                                  hipStream_t stream, float* ckpt = nullptr);

// With ckpt (backward checkpoints, ckpt_slot0 layout), runs the forward
// without outputs that stores every chunk's start state and the final state
// there instead (o, S_T unused).
hipError_t launch_fwd(const FwdPlan& plan, const void* q, const void* k, const void* v,
                      const void* alpha, const void* b, const void* w, int in_dtype,
                      const float* S0, void* o, int out_dtype, float* S_T,
                      const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int dk,
                      int dv, int gates, void* workspace, hipStream_t stream,
                      float* ckpt = nullptr);

// Backward (gate-aware chunked): device workspace bytes, and the launches
// (checkpoint forward, then the backward kernels of gdn2_bwd.hip).
size_t bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs, int in_dtype);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* alpha,
                      const void* b, const void* w, int in_dtype, const float* S0,
                      const void* dout, const float* dS_T, void* dq, void* dk, void* dv,
                      void* dalpha, void* db, void* dw, int grad_dtype, float* dS0,
                      const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int dkd,
                      int dvd, void* workspace, hipStream_t stream);

// Token-mixer prologue and epilogue (gdn2_mixer.hip).
hipError_t launch_prologue(const void* xq, const void* xk, const void* xv, const void* ga,
                           const void* gb, const void* gw, const float* Wq, const float* Wk,
                           const float* Wv, int K, float l2_eps, void* q, void* k, void* v,
                           void* alpha, void* b, void* w, const int32_t* cu, int nseq, int T,
                           int H, int64_t rows, int dk, int dv, int dtype, hipStream_t stream);
hipError_t launch_epilogue(const void* o, const void* g, const float* gamma, float eps, void* y,
                           int64_t nrows, int dv, int in_dtype, int out_dtype, hipStream_t stream);

}  // namespace gdn2
