// gdn2_api.hip -- the C ABI declared in include/gdn2.h: argument validation
// (before any launch), workspace sizing and dispatch to the kernels.
#include "gdn2.h"
#include "gdn2_internal.h"

namespace {

bool dims_ok(int32_t dk, int32_t dv) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

bool dtypes_ok(int32_t in_dtype, int32_t out_dtype) {
    if (in_dtype == GDN2_BF16) return out_dtype == GDN2_BF16 || out_dtype == GDN2_F32;
    if (in_dtype == GDN2_F32) return out_dtype == GDN2_F32;
    return false;
}

bool gates_ok(int32_t gates) {
    return gates == GDN2_GATES_FULL || gates == GDN2_GATES_KDA || gates == GDN2_GATES_GDN;
}

static_assert(GDN2_GATES_FULL == gdn2::GATES_FULL && GDN2_GATES_KDA == gdn2::GATES_KDA &&
                  GDN2_GATES_GDN == gdn2::GATES_GDN,
              "gate form values");

}  // namespace

extern "C" {

int gdn2_version(void) { return 2; }

const char* gdn2_status_string(int status) {
    switch (status) {
        case GDN2_OK: return "ok";
        case GDN2_ERR_INVALID_ARG: return "invalid argument";
        case GDN2_ERR_UNSUPPORTED: return "unsupported head size or dtype";
        case GDN2_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN2_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

size_t gdn2_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                               int32_t num_seqs, int32_t in_dtype) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 0 || !dims_ok(dk, dv)) return 0;
    if (in_dtype != GDN2_BF16 && in_dtype != GDN2_F32) return 0;
    return gdn2::plan_fwd(B, T, H, dk, dv, num_seqs, in_dtype).workspace;
}

int gdn2_fwd_gates(const void* q, const void* k, const void* v, const void* alpha,
                   const void* b, const void* w, int32_t gates, int32_t in_dtype, const float* S0,
                   void* o, int32_t out_dtype, float* S_T, const int32_t* cu_seqlens,
                   int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                   void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 1 || T < 0 || H < 1) return GDN2_ERR_INVALID_ARG;
    if (!gates_ok(gates)) return GDN2_ERR_INVALID_ARG;
    // one chunk of a token tensor (64 rows of H * d elements) is addressed
    // with 32-bit byte offsets
    if ((int64_t)H * (dk > dv ? dk : dv) >= ((int64_t)1 << 24)) return GDN2_ERR_INVALID_ARG;
    if (cu_seqlens && (B != 1 || num_seqs < 0)) return GDN2_ERR_INVALID_ARG;
    if (in_dtype != GDN2_BF16 && in_dtype != GDN2_F32) return GDN2_ERR_UNSUPPORTED;
    if (!dtypes_ok(in_dtype, out_dtype)) return GDN2_ERR_UNSUPPORTED;
    if (!dims_ok(dk, dv)) return GDN2_ERR_UNSUPPORTED;
    const int64_t N = cu_seqlens ? num_seqs : B;
    if (N * (int64_t)H > (int64_t)0x7fffffff / 2) return GDN2_ERR_INVALID_ARG;
    const bool have_tokens = (int64_t)B * T > 0;
    if (have_tokens && (!q || !k || !v || !alpha || !b || !w || !o)) return GDN2_ERR_INVALID_ARG;
    // o must not be any input buffer (a start-address check; partial
    // overlaps are the caller's responsibility)
    if (have_tokens && (o == q || o == k || o == v || o == alpha || o == b || o == w ||
                        o == static_cast<const void*>(S0) || o == static_cast<void*>(S_T)))
        return GDN2_ERR_INVALID_ARG;
    const gdn2::FwdPlan plan = gdn2::plan_fwd(B, T, H, dk, dv, num_seqs, in_dtype);
    if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace))
        return GDN2_ERR_WORKSPACE;
    const hipError_t e =
        gdn2::launch_fwd(plan, q, k, v, alpha, b, w, in_dtype, S0, o, out_dtype, S_T, cu_seqlens,
                         num_seqs, B, T, H, dk, dv, gates, workspace,
                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

int gdn2_fwd(const void* q, const void* k, const void* v, const void* alpha, const void* b,
             const void* w, int32_t in_dtype, const float* S0, void* o, int32_t out_dtype,
             float* S_T, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
             int32_t H, int32_t dk, int32_t dv, void* workspace, size_t workspace_bytes,
             void* stream) {
    return gdn2_fwd_gates(q, k, v, alpha, b, w, GDN2_GATES_FULL, in_dtype, S0, o, out_dtype, S_T,
                          cu_seqlens, num_seqs, B, T, H, dk, dv, workspace, workspace_bytes,
                          stream);
}

int gdn2_decode_gates(const void* q, const void* k, const void* v, const void* alpha,
                      const void* b, const void* w, int32_t gates, int32_t in_dtype, float* S,
                      void* o, int32_t out_dtype, int32_t N, int32_t H, int32_t dk, int32_t dv,
                      void* stream) {
    if (N < 0 || H < 1) return GDN2_ERR_INVALID_ARG;
    if (!gates_ok(gates)) return GDN2_ERR_INVALID_ARG;
    if (in_dtype != GDN2_BF16 && in_dtype != GDN2_F32) return GDN2_ERR_UNSUPPORTED;
    if (!dtypes_ok(in_dtype, out_dtype)) return GDN2_ERR_UNSUPPORTED;
    if (!dims_ok(dk, dv)) return GDN2_ERR_UNSUPPORTED;
    if (N == 0) return GDN2_OK;
    if ((int64_t)N * H * (dv / 32) > 0x7fffffff) return GDN2_ERR_INVALID_ARG;   // grid size
    if (!q || !k || !v || !alpha || !b || !w || !S || !o) return GDN2_ERR_INVALID_ARG;
    if (o == q || o == k || o == v || o == alpha || o == b || o == w || o == static_cast<void*>(S))
        return GDN2_ERR_INVALID_ARG;
    const hipError_t e = gdn2::launch_decode(q, k, v, alpha, b, w, in_dtype, S, o, out_dtype, N,
                                             H, dk, dv, gates, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

int gdn2_decode(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                const void* w, int32_t in_dtype, float* S, void* o, int32_t out_dtype, int32_t N,
                int32_t H, int32_t dk, int32_t dv, void* stream) {
    return gdn2_decode_gates(q, k, v, alpha, b, w, GDN2_GATES_FULL, in_dtype, S, o, out_dtype, N,
                             H, dk, dv, stream);
}

}  // extern "C"
