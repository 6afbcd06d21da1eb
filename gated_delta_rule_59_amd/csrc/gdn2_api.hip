// gdn2_api.hip -- the C ABI declared in include/gdn2.h: argument validation
// (before any launch), workspace sizing and dispatch to the kernels.
#include "gdn2.h"
#include "gdn2_internal.h"

#include <mutex>

// Device scratch of gdn2_fwd_noalloc: a file-scope device array, so the call
// never allocates.  Each GPU the library runs on holds its own copy until the
// process ends; its device address is looked up once per device (the name
// itself is only a host-side stand-in and must never reach a kernel).
static __device__ __align__(256) unsigned char scratch[GDN2_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES];   // device address of `scratch` per device, or null

// The current device's address of `scratch` (looked up on the first call on
// that device, with it current).  Returns null on any HIP error.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lk(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        scratch_ptr[dev] = p;
    }
    return scratch_ptr[dev];
}

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

// Argument checks of the forward entry points (everything except the
// workspace), and the launch plan.  No device call.
int check_fwd(const void* q, const void* k, const void* v, const void* alpha, const void* b,
              const void* w, int32_t gates, int32_t in_dtype, const float* S0, void* o,
              int32_t out_dtype, float* S_T, const int32_t* cu_seqlens, int32_t num_seqs,
              int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, gdn2::FwdPlan& plan) {
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
    // a dense batch has B sequences whatever num_seqs says
    plan = gdn2::plan_fwd(B, T, H, dk, dv, cu_seqlens ? num_seqs : B, in_dtype);
    return GDN2_OK;
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
    gdn2::FwdPlan plan;
    const int st = check_fwd(q, k, v, alpha, b, w, gates, in_dtype, S0, o, out_dtype, S_T,
                             cu_seqlens, num_seqs, B, T, H, dk, dv, plan);
    if (st != GDN2_OK) return st;
    if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace))
        return GDN2_ERR_WORKSPACE;
    const hipError_t e =
        gdn2::launch_fwd(plan, q, k, v, alpha, b, w, in_dtype, S0, o, out_dtype, S_T, cu_seqlens,
                         num_seqs, B, T, H, dk, dv, gates, workspace,
                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

int gdn2_fwd_ex(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                const void* w, int32_t gates, int32_t erase, int32_t in_dtype, const float* S0,
                void* o, int32_t out_dtype, float* S_T, const int32_t* cu_seqlens,
                int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                void* workspace, size_t workspace_bytes, void* stream) {
    if (erase == GDN2_ERASE_READ)
        return gdn2_fwd_gates(q, k, v, alpha, b, w, gates, in_dtype, S0, o, out_dtype, S_T,
                              cu_seqlens, num_seqs, B, T, H, dk, dv, workspace, workspace_bytes,
                              stream);
    if (erase != GDN2_ERASE_ROWS) return GDN2_ERR_INVALID_ARG;
    gdn2::FwdPlan plan;
    const int st = check_fwd(q, k, v, alpha, b, w, gates, in_dtype, S0, o, out_dtype, S_T,
                             cu_seqlens, num_seqs, B, T, H, dk, dv, plan);
    if (st != GDN2_OK) return st;
    if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace))
        return GDN2_ERR_WORKSPACE;
    const int N = cu_seqlens ? num_seqs : B;
    if (N == 0 || ((int64_t)B * T == 0 && S_T == nullptr)) return GDN2_OK;
    // token by token, split into segments under the same plan as the chunked
    // forward when the sequences are long and few
    const hipError_t e = gdn2::launch_fwd_serial_plan(plan, q, k, v, alpha, b, w, in_dtype, S0, o,
                                                      out_dtype, S_T, cu_seqlens, N, T, H, dk, dv,
                                                      gates, true, workspace,
                                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

int gdn2_fwd_noalloc(const void* q, const void* k, const void* v, const void* alpha,
                     const void* b, const void* w, int32_t gates, int32_t in_dtype,
                     const float* S0, void* o, int32_t out_dtype, float* S_T,
                     const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                     int32_t H, int32_t dk, int32_t dv, void* stream) {
    gdn2::FwdPlan plan;
    const int st = check_fwd(q, k, v, alpha, b, w, gates, in_dtype, S0, o, out_dtype, S_T,
                             cu_seqlens, num_seqs, B, T, H, dk, dv, plan);
    if (st != GDN2_OK) return st;
    // the token-serial forward (fp32 at dk = 128) also runs unsegmented,
    // without any workspace, when its segmented plan does not fit
    if (plan.workspace > GDN2_NOALLOC_SCRATCH_BYTES && in_dtype == GDN2_F32 && dk == 128) {
        plan.nseg = 1;
        plan.workspace = 0;
    }
    // the size check comes before anything touches the device
    if (plan.workspace > GDN2_NOALLOC_SCRATCH_BYTES) return GDN2_ERR_WORKSPACE;
    void* ws = nullptr;
    if (plan.workspace > 0 && !(ws = device_scratch())) return GDN2_ERR_HIP;
    const hipError_t e =
        gdn2::launch_fwd(plan, q, k, v, alpha, b, w, in_dtype, S0, o, out_dtype, S_T, cu_seqlens,
                         num_seqs, B, T, H, dk, dv, gates, ws, static_cast<hipStream_t>(stream));
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

size_t gdn2_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                               int32_t num_seqs, int32_t in_dtype) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 0 || !dims_ok(dk, dv)) return 0;
    if (in_dtype != GDN2_BF16 && in_dtype != GDN2_F32) return 0;
    return gdn2::bwd_workspace_bytes(B, T, H, dk, dv, num_seqs, in_dtype);
}

int gdn2_bwd(const void* q, const void* k, const void* v, const void* alpha, const void* b,
             const void* w, int32_t in_dtype, const float* S0, const void* dout,
             const float* dS_T, void* dq, void* dk_, void* dv_, void* dalpha, void* db, void* dw,
             int32_t grad_dtype, float* dS0, const int32_t* cu_seqlens, int32_t num_seqs,
             int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, void* workspace,
             size_t workspace_bytes, void* stream) {
    gdn2::FwdPlan plan;
    // the forward's checks (o stands for the gradient buffers: none may alias an input)
    const bool have_tokens = (int64_t)B * T > 0;
    int st = check_fwd(q, k, v, alpha, b, w, GDN2_GATES_FULL, in_dtype, S0,
                       have_tokens ? dq : nullptr, grad_dtype, nullptr, cu_seqlens, num_seqs, B,
                       T, H, dk, dv, plan);
    if (st != GDN2_OK) return st;
    if (have_tokens) {
        if (!dout || !dk_ || !dv_ || !dalpha || !db || !dw) return GDN2_ERR_INVALID_ARG;
        const void* ins[] = {q, k, v, alpha, b, w, dout, S0, dS_T};
        const void* outs[] = {dq, dk_, dv_, dalpha, db, dw, dS0};
        for (const void* o : outs)
            for (const void* i : ins)
                if (o && o == i) return GDN2_ERR_INVALID_ARG;
        for (int x = 0; x < 7; ++x)
            for (int y = x + 1; y < 7; ++y)
                if (outs[x] && outs[x] == outs[y]) return GDN2_ERR_INVALID_ARG;
    }
    const int32_t nseq = cu_seqlens ? num_seqs : B;   // a dense batch has B sequences
    const size_t need = gdn2::bwd_workspace_bytes(B, T, H, dk, dv, nseq, in_dtype);
    if (!workspace || workspace_bytes < need) return GDN2_ERR_WORKSPACE;
    const hipError_t e = gdn2::launch_bwd(q, k, v, alpha, b, w, in_dtype, S0, dout, dS_T, dq, dk_,
                                          dv_, dalpha, db, dw, grad_dtype, dS0, cu_seqlens,
                                          nseq, B, T, H, dk, dv, workspace,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

int gdn2_prologue(const void* xq, const void* xk, const void* xv, const void* ga,
                  const void* gb, const void* gw, const float* conv_q, const float* conv_k,
                  const float* conv_v, int32_t conv_width, float l2_eps, void* q, void* k,
                  void* v, void* alpha, void* b, void* w, const int32_t* cu_seqlens,
                  int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                  int32_t dtype, void* stream) {
    if (B < 1 || T < 0 || H < 1) return GDN2_ERR_INVALID_ARG;
    if (cu_seqlens && (B != 1 || num_seqs < 1)) return GDN2_ERR_INVALID_ARG;
    if (conv_width < 1 || conv_width > 4 || !(l2_eps >= 0.f)) return GDN2_ERR_INVALID_ARG;
    // a run of up to 12 rows is addressed with 32-bit byte offsets
    if ((int64_t)H * (dk > dv ? dk : dv) >= ((int64_t)1 << 24)) return GDN2_ERR_INVALID_ARG;
    if (dtype != GDN2_BF16 && dtype != GDN2_F32) return GDN2_ERR_UNSUPPORTED;
    if (!dims_ok(dk, dv)) return GDN2_ERR_UNSUPPORTED;
    const int64_t rows = (int64_t)B * T;
    if (rows == 0) return GDN2_OK;
    const void* ins[] = {xq, xk, xv, ga, gb, gw, conv_q, conv_k, conv_v};
    const void* outs[] = {q, k, v, alpha, b, w};
    for (const void* x : ins)
        if (!x) return GDN2_ERR_INVALID_ARG;
    for (int x = 0; x < 6; ++x) {
        if (!outs[x]) return GDN2_ERR_INVALID_ARG;
        for (const void* i : ins)
            if (outs[x] == i) return GDN2_ERR_INVALID_ARG;
        for (int y = x + 1; y < 6; ++y)
            if (outs[x] == outs[y]) return GDN2_ERR_INVALID_ARG;
    }
    const hipError_t e = gdn2::launch_prologue(
        xq, xk, xv, ga, gb, gw, conv_q, conv_k, conv_v, conv_width, l2_eps, q, k, v, alpha, b, w,
        cu_seqlens, cu_seqlens ? num_seqs : B, T, H, rows, dk, dv, dtype,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

int gdn2_epilogue(const void* o, const void* g, const float* gamma, float eps, void* y,
                  int32_t rows, int32_t H, int32_t dv, int32_t in_dtype, int32_t out_dtype,
                  void* stream) {
    if (rows < 0 || H < 1 || !(eps >= 0.f)) return GDN2_ERR_INVALID_ARG;
    if (!dtypes_ok(in_dtype, out_dtype)) return GDN2_ERR_UNSUPPORTED;
    if (dv != 64 && dv != 128) return GDN2_ERR_UNSUPPORTED;
    if (rows == 0) return GDN2_OK;
    if (!o || !g || !y || y == o || y == g) return GDN2_ERR_INVALID_ARG;
    const hipError_t e = gdn2::launch_epilogue(o, g, gamma, eps, y, (int64_t)rows * H, dv,
                                               in_dtype, out_dtype,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

int gdn2_decode_ex(const void* q, const void* k, const void* v, const void* alpha,
                   const void* b, const void* w, int32_t gates, int32_t erase, int32_t in_dtype,
                   float* S, void* o, int32_t out_dtype, int32_t N, int32_t H, int32_t dk,
                   int32_t dv, void* stream) {
    if (erase != GDN2_ERASE_READ && erase != GDN2_ERASE_ROWS) return GDN2_ERR_INVALID_ARG;
    if (N < 0 || H < 1) return GDN2_ERR_INVALID_ARG;
    if (!gates_ok(gates)) return GDN2_ERR_INVALID_ARG;
    if (in_dtype != GDN2_BF16 && in_dtype != GDN2_F32) return GDN2_ERR_UNSUPPORTED;
    if (!dtypes_ok(in_dtype, out_dtype)) return GDN2_ERR_UNSUPPORTED;
    if (!dims_ok(dk, dv)) return GDN2_ERR_UNSUPPORTED;
    if (N == 0) return GDN2_OK;
    // one workgroup per (sequence, head): the grid must fit 2^31 - 1
    const int64_t pairs = (int64_t)N * H;   // < 2^62
    if (pairs > (int64_t)0x7fffffff) return GDN2_ERR_INVALID_ARG;
    if (!q || !k || !v || !alpha || !b || !w || !S || !o) return GDN2_ERR_INVALID_ARG;
    if (o == q || o == k || o == v || o == alpha || o == b || o == w || o == static_cast<void*>(S))
        return GDN2_ERR_INVALID_ARG;
    const hipError_t e = gdn2::launch_decode(q, k, v, alpha, b, w, in_dtype, S, o, out_dtype, N,
                                             H, dk, dv, gates, static_cast<hipStream_t>(stream),
                                             erase == GDN2_ERASE_ROWS);
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

int gdn2_decode_gates(const void* q, const void* k, const void* v, const void* alpha,
                      const void* b, const void* w, int32_t gates, int32_t in_dtype, float* S,
                      void* o, int32_t out_dtype, int32_t N, int32_t H, int32_t dk, int32_t dv,
                      void* stream) {
    return gdn2_decode_ex(q, k, v, alpha, b, w, gates, GDN2_ERASE_READ, in_dtype, S, o, out_dtype,
                          N, H, dk, dv, stream);
}

int gdn2_decode(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                const void* w, int32_t in_dtype, float* S, void* o, int32_t out_dtype, int32_t N,
                int32_t H, int32_t dk, int32_t dv, void* stream) {
    return gdn2_decode_gates(q, k, v, alpha, b, w, GDN2_GATES_FULL, in_dtype, S, o, out_dtype, N,
                             H, dk, dv, stream);
}

}  // extern "C"
