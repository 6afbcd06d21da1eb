// gdn2_mixer.hip -- the elementwise prologue and epilogue of the Gated
// DeltaNet-2 token mixer around the recurrence (gfx950).
//
// Japanese article, "architecture and benchmarks", paragraph 1: q and k pass a
// short causal convolution, SiLU and an L2 normalisation per head-token; v a
// short convolution and SiLU; the decay, erase and write gates a sigmoid; the
// output an RMSNorm times a SiLU output gate.  The projections around them
// are matrix products outside this path.  Each kernel below is one pass over
// HBM: every input row read once, every output row written once, 16 bytes
// per lane.
//
//   gdn2_prologue_kernel:
//       q = L2norm(SiLU(conv_K(xq))), k = L2norm(SiLU(conv_K(xk))),
//       v = SiLU(conv_K(xv)), alpha, b, w = sigmoid(ga, gb, gw)
//     conv_K is the depthwise causal convolution of width K <= 4 within the
//     row's sequence (earlier tokens of the sequence only).
//   gdn2_epilogue_kernel, per (token, head) row:
//       y = o / sqrt(mean(o^2) + eps) * gamma * SiLU(g)
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

constexpr int MX_THREADS = 256;
__device__ __forceinline__ float sigmoidf_(float y) { return 1.f / (1.f + __expf(-y)); }
__device__ __forceinline__ float siluf_(float y) { return y * sigmoidf_(y); }
}  // namespace

// Prologue work split: thread (run, tensor, head, channel group) walks the
// MX_RUN tokens of its run for 8 channels of one of q, k, v (and the gate
// that shares their width: alpha with q, b with k, w with v).  Its
// convolution taps stay in registers and the K - 1 previous inputs in a
// sliding window, so each input row is read from HBM once, with one 16-byte
// load per lane; the rows of the next two tokens are loaded while the
// current one is computed.  Lane order: channel group fastest, then head, then tensor; each
// run starts on a wave boundary.  The L2 norm of a q or k row sums over its
// DK/8 lanes, an aligned group inside one wave.
constexpr int MX_RUN = 64;

__device__ __forceinline__ void st8(bf16_t* p, const float (&x)[8]) {
    uint4 u;
    u.x = f32x2_to_bf16x2(x[0], x[1]);
    u.y = f32x2_to_bf16x2(x[2], x[3]);
    u.z = f32x2_to_bf16x2(x[4], x[5]);
    u.w = f32x2_to_bf16x2(x[6], x[7]);
    *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void st8(float* p, const float (&x)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}
// sum over the aligned group of G lanes that holds this lane
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = 1; o < G; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// lanes per run of the prologue: H (2 DK/8 + DV/8), rounded up to a wave
__host__ __device__ __forceinline__ int prologue_run_lanes(int H, int dk, int dv) {
    return (H * (2 * (dk / 8) + dv / 8) + 63) / 64 * 64;
}

template <typename In, int DK, int DV, int K>
__global__ __launch_bounds__(MX_THREADS) void gdn2_prologue_kernel(
    const In* __restrict__ xq, const In* __restrict__ xk, const In* __restrict__ xv,
    const In* __restrict__ ga, const In* __restrict__ gb, const In* __restrict__ gw,
    const float* __restrict__ Wq, const float* __restrict__ Wk, const float* __restrict__ Wv,
    float l2_eps, In* __restrict__ q, In* __restrict__ k, In* __restrict__ v,
    In* __restrict__ alpha, In* __restrict__ b, In* __restrict__ w, const int32_t* __restrict__ cu,
    int nseq, int T, int H, int64_t rows) {
    constexpr int GK = DK / 8, GV = DV / 8;
    const int per_run = prologue_run_lanes(H, DK, DV);
    const int64_t gid = (int64_t)blockIdx.x * MX_THREADS + threadIdx.x;
    const int64_t run = gid / per_run;
    const int idx = (int)(gid - run * per_run);
    const int nk = H * GK;
    // tensor j (0 q, 1 k, 2 v; 3: a padding lane), head h, channel group c
    int j, h, c;
    if (idx < 2 * nk) {
        j = idx < nk ? 0 : 1;
        const int r = idx - j * nk;
        h = r / GK;
        c = r - h * GK;
    } else {
        const int r = idx - 2 * nk;
        h = r / GV;
        c = r - h * GV;
        j = h < H ? 2 : 3;
    }
    const int64_t t0 = run * MX_RUN;
    if (t0 >= rows) return;   // whole waves: a run starts on a wave boundary
    const int64_t t1 = t0 + MX_RUN < rows ? t0 + MX_RUN : rows;
    const bool active = j < 3;
    const int D = j < 2 ? DK : DV;
    const In* const x = j == 0 ? xq : j == 1 ? xk : xv;
    const In* const g = j == 0 ? ga : j == 1 ? gb : gw;
    In* const y = j == 0 ? q : j == 1 ? k : v;
    In* const gy = j == 0 ? alpha : j == 1 ? b : w;
    const float* const Wt = j == 0 ? Wq : j == 1 ? Wk : Wv;
    const size_t stride = (size_t)H * D;
    const size_t off = (size_t)h * D + 8 * c;
    float taps[K][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int jj = 0; jj < K; ++jj) taps[jj][i] = active ? Wt[(off + i) * K + jj] : 0.f;
    // sequence of t0: [sstart, snext); packed: the last sequence starting at
    // or before t0 (empty sequences skipped)
    int s = 0;
    int64_t sstart, snext;
    if (cu) {
        int lo = 0, hi = nseq - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu[mid] <= t0) lo = mid;
            else hi = mid - 1;
        }
        s = lo;
        sstart = cu[s];
        snext = cu[s + 1];
    } else {
        sstart = t0 - t0 % T;
        snext = sstart + T;
    }
    // window: inputs of tokens t - K + 1 .. t - 1 (zero before the sequence)
    float win[K > 1 ? K - 1 : 1][8];
#pragma unroll
    for (int jj = 0; jj < K - 1; ++jj) {
        const int64_t tok = t0 - (K - 1) + jj;
        if (active && tok >= sstart) load8(x + (size_t)tok * stride + off, win[jj]);
        else
#pragma unroll
            for (int i = 0; i < 8; ++i) win[jj][i] = 0.f;
    }
    // rows of tokens t (cx, cg), t + 1 and t + 2 (loaded ahead)
    float cx[8] = {}, cg[8] = {}, x1[8] = {}, g1[8] = {};
    if (active) {
        load8(x + (size_t)t0 * stride + off, cx);
        load8(g + (size_t)t0 * stride + off, cg);
        if (t0 + 1 < t1) {
            load8(x + (size_t)(t0 + 1) * stride + off, x1);
            load8(g + (size_t)(t0 + 1) * stride + off, g1);
        }
    }
    for (int64_t t = t0; t < t1; ++t) {
        float x2[8] = {}, g2[8] = {};
        if (active && t + 2 < t1) {
            load8(x + (size_t)(t + 2) * stride + off, x2);
            load8(g + (size_t)(t + 2) * stride + off, g2);
        }
        if (t == snext) {   // a sequence starts at t: no history
            if (cu) {
                while (s < nseq - 1 && cu[s + 1] <= t) ++s;
                snext = cu[s + 1];
            } else {
                snext += T;
            }
#pragma unroll
            for (int jj = 0; jj < K - 1; ++jj)
#pragma unroll
                for (int i = 0; i < 8; ++i) win[jj][i] = 0.f;
        }
        float yv[8];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int jj = 0; jj < K - 1; ++jj) acc = fmaf(taps[jj][i], win[jj][i], acc);
            acc = fmaf(taps[K - 1][i], cx[i], acc);
            yv[i] = siluf_(acc);
            ss = fmaf(yv[i], yv[i], ss);
        }
        ss = group_sum<GK>(ss);
        if (j < 2) {
            const float r = 1.f / sqrtf(ss + l2_eps);
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] *= r;
        }
        if (active) {
#pragma unroll
            for (int i = 0; i < 8; ++i) cg[i] = sigmoidf_(cg[i]);
            st8(y + (size_t)t * stride + off, yv);
            st8(gy + (size_t)t * stride + off, cg);
        }
#pragma unroll
        for (int jj = 0; jj + 1 < K - 1; ++jj)
#pragma unroll
            for (int i = 0; i < 8; ++i) win[jj][i] = win[jj + 1][i];
        if constexpr (K > 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) win[K - 2][i] = cx[i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            cx[i] = x1[i];
            cg[i] = g1[i];
            x1[i] = x2[i];
            g1[i] = g2[i];
        }
    }
}

// Epilogue: thread (row, channel group) with DV/8 lanes per (token, head)
// row, grid-stride over rows; the rows two strides ahead are loaded while
// the current one is computed.
template <typename In, typename Out, int DV>
__global__ __launch_bounds__(MX_THREADS) void gdn2_epilogue_kernel(
    const In* __restrict__ o, const In* __restrict__ g, const float* __restrict__ gamma, float eps,
    Out* __restrict__ y, int64_t nrows) {
    constexpr int G = DV / 8;
    const int64_t gid = (int64_t)blockIdx.x * MX_THREADS + threadIdx.x;
    const int c = (int)(gid % G);
    const int64_t step = ((int64_t)gridDim.x * MX_THREADS) / G;
    float gm[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) gm[i] = gamma ? gamma[8 * c + i] : 1.f;
    // rows row (x, gg), row + step and row + 2 step (loaded ahead)
    int64_t row = gid / G;
    float x[8] = {}, gg[8] = {}, x1[8] = {}, g1[8] = {};
    if (row < nrows) {
        load8(o + (size_t)row * DV + 8 * c, x);
        load8(g + (size_t)row * DV + 8 * c, gg);
    }
    if (row + step < nrows) {
        load8(o + (size_t)(row + step) * DV + 8 * c, x1);
        load8(g + (size_t)(row + step) * DV + 8 * c, g1);
    }
    for (; row < nrows; row += step) {
        float x2[8] = {}, g2[8] = {};
        const int64_t nr = row + 2 * step;
        if (nr < nrows) {
            load8(o + (size_t)nr * DV + 8 * c, x2);
            load8(g + (size_t)nr * DV + 8 * c, g2);
        }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
        ss = group_sum<G>(ss);
        const float r = 1.f / sqrtf(ss / DV + eps);
        float out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = x[i] * r * gm[i] * siluf_(gg[i]);
        st8(y + (size_t)row * DV + 8 * c, out);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = x1[i];
            gg[i] = g1[i];
            x1[i] = x2[i];
            g1[i] = g2[i];
        }
    }
}

namespace {

unsigned mx_grid(int64_t threads_needed) {
    // at most 16 workgroups per compute unit; the epilogue strides
    const int64_t wg = (threads_needed + MX_THREADS - 1) / MX_THREADS;
    const int64_t cap = 256 * 16;
    return (unsigned)(wg < 1 ? 1 : (wg < cap ? wg : cap));
}

template <typename In, int DK, int DV>
hipError_t launch_prologue_d(const void* xq, const void* xk, const void* xv, const void* ga,
                             const void* gb, const void* gw, const float* Wq, const float* Wk,
                             const float* Wv, int K, float l2_eps, void* q, void* k, void* v,
                             void* alpha, void* b, void* w, const int32_t* cu, int nseq, int T,
                             int H, int64_t rows, hipStream_t stream) {
    // one thread per (run, lane of the run): every run is covered
    const int64_t nruns = (rows + MX_RUN - 1) / MX_RUN;
    const int64_t threads = nruns * prologue_run_lanes(H, DK, DV);
    if ((threads + MX_THREADS - 1) / MX_THREADS > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((threads + MX_THREADS - 1) / MX_THREADS));
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
    const dim3 grid(mx_grid(nrows * (dv / 8)));
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
