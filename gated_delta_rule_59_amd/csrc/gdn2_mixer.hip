// gdn2_mixer.hip -- the elementwise prologue and epilogue of the Gated
// DeltaNet-2 token mixer around the recurrence (gfx950).
//
// Japanese article, "architecture and benchmarks", paragraph 1: q and k pass a
// short causal convolution, SiLU and an L2 normalisation per head-token; v a
// short convolution and SiLU; the decay, erase and write gates a sigmoid; the
// output an RMSNorm times a SiLU output gate.  The projections around them
// are matrix products outside this path.  Each kernel below is one pass over
// HBM: every input row read once from HBM (the convolution's earlier rows
// come back from the L2), every output row written once.
//
//   gdn2_prologue_kernel: one wave per (token, head) row at a time (grid-
//     stride over rows); lane l holds channels CK l .. CK l + CK - 1.
//       q = L2norm(SiLU(conv_K(xq))), k = L2norm(SiLU(conv_K(xk))),
//       v = SiLU(conv_K(xv)), alpha, b, w = sigmoid(ga, gb, gw)
//     conv_K is the depthwise causal convolution of width K <= 4 within the
//     row's sequence (earlier tokens of the sequence only).
//   gdn2_epilogue_kernel: one wave per (token, head) row:
//       y = o / sqrt(mean(o^2) + eps) * gamma * SiLU(g)
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

constexpr int MX_THREADS = 256;
constexpr int MX_KMAX = 4;

__device__ __forceinline__ float mx_ld(const bf16_t* p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ float mx_ld(const float* p) { return *p; }

template <int N, typename T> struct Vec;
template <> struct Vec<1, bf16_t> {
    static __device__ __forceinline__ void ld(const bf16_t* p, float (&x)[1]) { x[0] = mx_ld(p); }
    static __device__ __forceinline__ void st(bf16_t* p, const float (&x)[1]) { store1(p, x[0]); }
};
template <> struct Vec<2, bf16_t> {
    static __device__ __forceinline__ void ld(const bf16_t* p, float (&x)[2]) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
        x[0] = bf16_to_f32((uint16_t)(u & 0xffff));
        x[1] = bf16_to_f32((uint16_t)(u >> 16));
    }
    static __device__ __forceinline__ void st(bf16_t* p, const float (&x)[2]) {
        *reinterpret_cast<uint32_t*>(p) = f32x2_to_bf16x2(x[0], x[1]);
    }
};
template <> struct Vec<1, float> {
    static __device__ __forceinline__ void ld(const float* p, float (&x)[1]) { x[0] = *p; }
    static __device__ __forceinline__ void st(float* p, const float (&x)[1]) { *p = x[0]; }
};
template <> struct Vec<2, float> {
    static __device__ __forceinline__ void ld(const float* p, float (&x)[2]) {
        const float2 u = *reinterpret_cast<const float2*>(p);
        x[0] = u.x;
        x[1] = u.y;
    }
    static __device__ __forceinline__ void st(float* p, const float (&x)[2]) {
        *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
    }
};

__device__ __forceinline__ float sigmoidf_(float y) { return 1.f / (1.f + __expf(-y)); }
__device__ __forceinline__ float siluf_(float y) { return y * sigmoidf_(y); }
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// token index within its sequence (dense rows: tok % T; packed: by binary
// search over cu_seqlens)
__device__ __forceinline__ int64_t pos_in_seq(int64_t tok, const int32_t* cu, int nseq, int T) {
    if (!cu) return tok % T;
    int lo = 0, hi = nseq - 1;   // last sequence starting at or before tok
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= tok) lo = mid;
        else hi = mid - 1;
    }
    return tok - cu[lo];
}

}  // namespace

template <typename In, int DK, int DV, int K>
__global__ __launch_bounds__(MX_THREADS) void gdn2_prologue_kernel(
    const In* __restrict__ xq, const In* __restrict__ xk, const In* __restrict__ xv,
    const In* __restrict__ ga, const In* __restrict__ gb, const In* __restrict__ gw,
    const float* __restrict__ Wq, const float* __restrict__ Wk, const float* __restrict__ Wv,
    float l2_eps, In* __restrict__ q, In* __restrict__ k, In* __restrict__ v,
    In* __restrict__ alpha, In* __restrict__ b, In* __restrict__ w, const int32_t* __restrict__ cu,
    int nseq, int T, int H, int64_t rows) {
    constexpr int CK = DK / 64, CV = DV / 64;
    const int lane = threadIdx.x & 63;
    const int64_t wave0 = ((int64_t)blockIdx.x * MX_THREADS + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * MX_THREADS) >> 6;
    for (int64_t row = wave0; row < rows * H; row += nwaves) {   // row = token * H + head
        const int64_t tok = row / H;
        const int h = (int)(row - tok * H);
        const int64_t pos = pos_in_seq(tok, cu, nseq, T);
        const size_t kst = (size_t)H * DK, vst = (size_t)H * DV;
        const size_t ko = (size_t)row * DK + CK * lane, vo = (size_t)row * DV + CV * lane;
        // convolution over the row's sequence: rows tok - K + 1 + j with
        // pos - K + 1 + j >= 0
        float yq[CK] = {}, yk[CK] = {}, yv[CV] = {};
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int back = K - 1 - j;
            if (pos < back) continue;
            float a[CK], c[CK], e[CV];
            Vec<CK, In>::ld(xq + ko - (size_t)back * kst, a);
            Vec<CK, In>::ld(xk + ko - (size_t)back * kst, c);
            Vec<CV, In>::ld(xv + vo - (size_t)back * vst, e);
#pragma unroll
            for (int u = 0; u < CK; ++u) {
                const size_t ch = (size_t)h * DK + CK * lane + u;
                yq[u] += Wq[ch * K + j] * a[u];
                yk[u] += Wk[ch * K + j] * c[u];
            }
#pragma unroll
            for (int u = 0; u < CV; ++u) yv[u] += Wv[((size_t)h * DV + CV * lane + u) * K + j] * e[u];
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int u = 0; u < CK; ++u) {
            yq[u] = siluf_(yq[u]);
            yk[u] = siluf_(yk[u]);
            sq += yq[u] * yq[u];
            sk += yk[u] * yk[u];
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        const float rq = 1.f / sqrtf(sq + l2_eps), rk = 1.f / sqrtf(sk + l2_eps);
#pragma unroll
        for (int u = 0; u < CK; ++u) {
            yq[u] *= rq;
            yk[u] *= rk;
        }
#pragma unroll
        for (int u = 0; u < CV; ++u) yv[u] = siluf_(yv[u]);
        Vec<CK, In>::st(q + ko, yq);
        Vec<CK, In>::st(k + ko, yk);
        Vec<CV, In>::st(v + vo, yv);
        float a[CK], c[CK], e[CV];
        Vec<CK, In>::ld(ga + ko, a);
        Vec<CK, In>::ld(gb + ko, c);
        Vec<CV, In>::ld(gw + vo, e);
#pragma unroll
        for (int u = 0; u < CK; ++u) {
            a[u] = sigmoidf_(a[u]);
            c[u] = sigmoidf_(c[u]);
        }
#pragma unroll
        for (int u = 0; u < CV; ++u) e[u] = sigmoidf_(e[u]);
        Vec<CK, In>::st(alpha + ko, a);
        Vec<CK, In>::st(b + ko, c);
        Vec<CV, In>::st(w + vo, e);
    }
}

template <typename In, typename Out, int DV>
__global__ __launch_bounds__(MX_THREADS) void gdn2_epilogue_kernel(
    const In* __restrict__ o, const In* __restrict__ g, const float* __restrict__ gamma, float eps,
    Out* __restrict__ y, int64_t nrows) {
    constexpr int CV = DV / 64;
    const int lane = threadIdx.x & 63;
    const int64_t wave0 = ((int64_t)blockIdx.x * MX_THREADS + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * MX_THREADS) >> 6;
    for (int64_t row = wave0; row < nrows; row += nwaves) {
        const size_t off = (size_t)row * DV + CV * lane;
        float x[CV], gg[CV];
        Vec<CV, In>::ld(o + off, x);
        Vec<CV, In>::ld(g + off, gg);
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < CV; ++u) ss += x[u] * x[u];
        ss = wave_sum(ss);
        const float r = 1.f / sqrtf(ss / DV + eps);
        float out[CV];
#pragma unroll
        for (int u = 0; u < CV; ++u) {
            const float gm = gamma ? gamma[CV * lane + u] : 1.f;
            out[u] = x[u] * r * gm * siluf_(gg[u]);
        }
        Vec<CV, Out>::st(y + off, out);
    }
}

namespace {

unsigned mx_grid(int64_t waves_needed) {
    // enough workgroups to fill the chip several times; the kernels stride
    const int64_t wg = (waves_needed + 3) / 4;
    const int64_t cap = 256 * 16;
    return (unsigned)(wg < 1 ? 1 : (wg < cap ? wg : cap));
}

template <typename In, int DK, int DV>
hipError_t launch_prologue_d(const void* xq, const void* xk, const void* xv, const void* ga,
                             const void* gb, const void* gw, const float* Wq, const float* Wk,
                             const float* Wv, int K, float l2_eps, void* q, void* k, void* v,
                             void* alpha, void* b, void* w, const int32_t* cu, int nseq, int T,
                             int H, int64_t rows, hipStream_t stream) {
    const dim3 grid(mx_grid(rows * H));
#define GDN2_PRO_ARGS                                                                           \
    static_cast<const In*>(xq), static_cast<const In*>(xk), static_cast<const In*>(xv),         \
        static_cast<const In*>(ga), static_cast<const In*>(gb), static_cast<const In*>(gw), Wq, \
        Wk, Wv, l2_eps, static_cast<In*>(q), static_cast<In*>(k), static_cast<In*>(v),          \
        static_cast<In*>(alpha), static_cast<In*>(b), static_cast<In*>(w), cu, nseq, T, H, rows
    switch (K) {
        case 1: hipLaunchKernelGGL((gdn2_prologue_kernel<In, DK, DV, 1>), grid, dim3(MX_THREADS), 0, stream, GDN2_PRO_ARGS); break;
        case 2: hipLaunchKernelGGL((gdn2_prologue_kernel<In, DK, DV, 2>), grid, dim3(MX_THREADS), 0, stream, GDN2_PRO_ARGS); break;
        case 3: hipLaunchKernelGGL((gdn2_prologue_kernel<In, DK, DV, 3>), grid, dim3(MX_THREADS), 0, stream, GDN2_PRO_ARGS); break;
        default: hipLaunchKernelGGL((gdn2_prologue_kernel<In, DK, DV, 4>), grid, dim3(MX_THREADS), 0, stream, GDN2_PRO_ARGS); break;
    }
#undef GDN2_PRO_ARGS
    return hipGetLastError();
}

template <typename In>
hipError_t launch_prologue_t(const void* xq, const void* xk, const void* xv, const void* ga,
                             const void* gb, const void* gw, const float* Wq, const float* Wk,
                             const float* Wv, int K, float l2_eps, void* q, void* k, void* v,
                             void* alpha, void* b, void* w, const int32_t* cu, int nseq, int T,
                             int H, int64_t rows, int dk, int dv, hipStream_t stream) {
#define GDN2_PRO_CALL(DK_, DV_)                                                                 \
    return launch_prologue_d<In, DK_, DV_>(xq, xk, xv, ga, gb, gw, Wq, Wk, Wv, K, l2_eps, q, k, \
                                           v, alpha, b, w, cu, nseq, T, H, rows, stream)
    if (dk == 128 && dv == 128) GDN2_PRO_CALL(128, 128);
    if (dk == 128 && dv == 64) GDN2_PRO_CALL(128, 64);
    if (dk == 64 && dv == 128) GDN2_PRO_CALL(64, 128);
    GDN2_PRO_CALL(64, 64);
#undef GDN2_PRO_CALL
}

}  // namespace

hipError_t launch_prologue(const void* xq, const void* xk, const void* xv, const void* ga,
                           const void* gb, const void* gw, const float* Wq, const float* Wk,
                           const float* Wv, int K, float l2_eps, void* q, void* k, void* v,
                           void* alpha, void* b, void* w, const int32_t* cu, int nseq, int T,
                           int H, int64_t rows, int dk, int dv, int dtype, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if (dtype == DT_BF16)
        return launch_prologue_t<bf16_t>(xq, xk, xv, ga, gb, gw, Wq, Wk, Wv, K, l2_eps, q, k, v,
                                         alpha, b, w, cu, nseq, T, H, rows, dk, dv, stream);
    return launch_prologue_t<float>(xq, xk, xv, ga, gb, gw, Wq, Wk, Wv, K, l2_eps, q, k, v,
                                    alpha, b, w, cu, nseq, T, H, rows, dk, dv, stream);
}

hipError_t launch_epilogue(const void* o, const void* g, const float* gamma, float eps, void* y,
                           int64_t nrows, int dv, int in_dtype, int out_dtype, hipStream_t stream) {
    if (nrows == 0) return hipSuccess;
    const dim3 grid(mx_grid(nrows));
#define GDN2_EPI(IN_, OUT_, DV_)                                                                  \
    hipLaunchKernelGGL((gdn2_epilogue_kernel<IN_, OUT_, DV_>), grid, dim3(MX_THREADS), 0, stream, \
                       static_cast<const IN_*>(o), static_cast<const IN_*>(g), gamma, eps,        \
                       static_cast<OUT_*>(y), nrows)
    if (in_dtype == DT_BF16) {
        if (out_dtype == DT_BF16) {
            if (dv == 128) GDN2_EPI(bf16_t, bf16_t, 128); else GDN2_EPI(bf16_t, bf16_t, 64);
        } else {
            if (dv == 128) GDN2_EPI(bf16_t, float, 128); else GDN2_EPI(bf16_t, float, 64);
        }
    } else {
        if (dv == 128) GDN2_EPI(float, float, 128); else GDN2_EPI(float, float, 64);
    }
#undef GDN2_EPI
    return hipGetLastError();
}

}  // namespace gdn2
