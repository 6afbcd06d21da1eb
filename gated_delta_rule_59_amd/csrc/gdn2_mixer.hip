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
// 1 / (1 + e^-y) with the hardware reciprocal (about 1 ulp): an exact
// division would cost a ten-instruction sequence per element.  y -> -inf
// gives rcp(inf) = 0, y -> +inf gives 1.
__device__ __forceinline__ float sigmoidf_(float y) {
    return __builtin_amdgcn_rcpf(1.f + __expf(-y));
}
__device__ __forceinline__ float siluf_(float y) { return y * sigmoidf_(y); }
// hardware reciprocal square root (about 1 ulp)
__device__ __forceinline__ float rsqrt_(float y) { return __builtin_amdgcn_rsqf(y); }
}  // namespace

// Output rows are written once and read by a later kernel: non-temporal
// stores (the prologue measured 0.306 against 0.318 ms on the 1.3B-layer
// shape, the epilogue 1% less; the same hint on the forward's o stores made
// that kernel 11% slower back to back).
__device__ __forceinline__ void st8(bf16_t* p, const float (&x)[8]) {
    uint4 u;
    u.x = f32x2_to_bf16x2(x[0], x[1]);
    u.y = f32x2_to_bf16x2(x[2], x[3]);
    u.z = f32x2_to_bf16x2(x[4], x[5]);
    u.w = f32x2_to_bf16x2(x[6], x[7]);
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    const u4v uv = {u.x, u.y, u.z, u.w};
    __builtin_nontemporal_store(uv, reinterpret_cast<u4v*>(p));
}
__device__ __forceinline__ void st8(float* p, const float (&x)[8]) {
    const floatx4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<floatx4*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<floatx4*>(p + 4));
}
// sum over the aligned group of G lanes that holds this lane, by DPP moves
// inside the lane's 16-lane row (each step adds the partner that holds the
// other half of the group so far): a few cycles each, where a lane shuffle
// through the LDS crossbar (ds_bpermute) is a round trip of its own
template <int CTRL>
__device__ __forceinline__ float mx_dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ __forceinline__ float group_sum_dpp(float x) {
    static_assert(G == 2 || G == 4 || G == 8 || G == 16, "groups inside one DPP row");
    x += mx_dpp<0xB1>(x);                          // quad_perm [1,0,3,2]
    if constexpr (G >= 4) x += mx_dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    if constexpr (G >= 8) x += mx_dpp<0x141>(x);   // row_half_mirror
    if constexpr (G >= 16) x += mx_dpp<0x140>(x);  // row_mirror
    return x;
}
// the same by lane shuffles: the epilogue, where it measured 1% faster than
// the DPP form (one sum per row there, none of the prologue's row chain)
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = 1; o < G; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Prologue: thread (run, tensor, head, channel group) takes 8 channels of
// one of q, k, v (and of the gate that shares their width: alpha with q, b
// with k, w with v) for a run of RUN tokens.  It issues the loads of all its rows first
// (the K - 1 rows before the run, the run's inputs and gates, kept as raw
// storage words), then its convolution taps, and only then computes and
// stores the run row by row.  Many short runs keep far more loads in flight
// per compute unit than one long run with a two-row prefetch; the K - 1 rows
// before a run were read by the run before it and mostly come from L2.
// Each tensor's lanes of a run are padded to whole waves, so the tensor is
// uniform across a wave and its rows are addressed through buffer
// descriptors held in scalar registers: a row outside the descriptor's
// range (before the sequence, past the end) reads as zero and a store there
// is dropped, so neither needs a branch.
template <typename In>
struct Raw8;
template <>
struct Raw8<bf16_t> {
    uint4 u;
};
template <>
struct Raw8<float> {
    float4 a, b;
};
typedef uint32_t mx_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int64_t mx_uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ void ld_raw(__amdgpu_buffer_rsrc_t r, uint32_t off, Raw8<bf16_t>& x) {
    const mx_u32x4 u = __builtin_bit_cast(mx_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    x.u = make_uint4(u[0], u[1], u[2], u[3]);
}
__device__ __forceinline__ void ld_raw(__amdgpu_buffer_rsrc_t r, uint32_t off, Raw8<float>& x) {
    const mx_u32x4 u0 = __builtin_bit_cast(mx_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    const mx_u32x4 u1 = __builtin_bit_cast(mx_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off + 16, 0, 0));
    x.a = make_float4(__uint_as_float(u0[0]), __uint_as_float(u0[1]), __uint_as_float(u0[2]), __uint_as_float(u0[3]));
    x.b = make_float4(__uint_as_float(u1[0]), __uint_as_float(u1[1]), __uint_as_float(u1[2]), __uint_as_float(u1[3]));
}
__device__ __forceinline__ void widen(const Raw8<bf16_t>& r, float (&x)[8]) {
    uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
    // widen at the use: otherwise the compiler widens every row as soon as
    // it lands and holds twice the registers
    asm volatile("" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void widen(const Raw8<float>& r, float (&x)[8]) {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}
// (cache policy 2: non-temporal, as st8)
__device__ __forceinline__ void st_raw(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&x)[8],
                                       const bf16_t*) {
    const mx_u32x4 u = {f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3]),
                        f32x2_to_bf16x2(x[4], x[5]), f32x2_to_bf16x2(x[6], x[7])};
    __builtin_amdgcn_raw_buffer_store_b128(u, r, (int)off, 0, 2);
}
__device__ __forceinline__ void st_raw(__amdgpu_buffer_rsrc_t r, uint32_t off, const float (&x)[8],
                                       const float*) {
    const mx_u32x4 u0 = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    const mx_u32x4 u1 = {__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])};
    __builtin_amdgcn_raw_buffer_store_b128(u0, r, (int)off, 0, 2);
    __builtin_amdgcn_raw_buffer_store_b128(u1, r, (int)off + 16, 0, 2);
}

// lanes per run of the short-run prologue: the q, k and v sections, each
// rounded up to whole waves
__host__ __device__ __forceinline__ int prologue_short_run_lanes(int H, int dk, int dv) {
    return 2 * ((H * (dk / 8) + 63) & ~63) + ((H * (dv / 8) + 63) & ~63);
}

template <typename In, int DK, int DV, int K, int RUN>
__global__ __launch_bounds__(MX_THREADS) void gdn2_prologue_run_kernel(
    const In* __restrict__ xq, const In* __restrict__ xk, const In* __restrict__ xv,
    const In* __restrict__ ga, const In* __restrict__ gb, const In* __restrict__ gw,
    const float* __restrict__ Wq, const float* __restrict__ Wk, const float* __restrict__ Wv,
    float l2_eps, In* __restrict__ q, In* __restrict__ k, In* __restrict__ v,
    In* __restrict__ alpha, In* __restrict__ b, In* __restrict__ w, const int32_t* __restrict__ cu,
    int nseq, int T, int H, int64_t rows) {
    constexpr int GK = DK / 8, GV = DV / 8;
    const int nk = (H * GK + 63) & ~63;
    const int per_run = prologue_short_run_lanes(H, DK, DV);
    // a wave lies inside one run and one tensor section: everything but the
    // lane's head and channel group is uniform across it (scalar registers)
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t gid0 = (int64_t)blockIdx.x * MX_THREADS + 64 * wave;
    const int64_t run = gid0 / per_run;
    const int idx0 = (int)(gid0 - run * per_run);
    const int j = idx0 < nk ? 0 : idx0 < 2 * nk ? 1 : 2;
    const int lidx = idx0 - j * nk + (int)(threadIdx.x & 63);
    const int G = j < 2 ? GK : GV;
    const int h = lidx / G;
    const int c = lidx - h * G;
    const int64_t t0 = run * RUN;
    if (t0 >= rows) return;
    const int nr = (int)(rows - t0 < RUN ? rows - t0 : RUN);
    const bool active = h < H;
    const int D = j < 2 ? DK : DV;
    const In* const x = j == 0 ? xq : j == 1 ? xk : xv;
    const In* const g = j == 0 ? ga : j == 1 ? gb : gw;
    In* const y = j == 0 ? q : j == 1 ? k : v;
    In* const gy = j == 0 ? alpha : j == 1 ? b : w;
    const float* const Wt = j == 0 ? Wq : j == 1 ? Wk : Wv;
    const int64_t stride = (int64_t)H * D;
    const uint32_t rowb = (uint32_t)(stride * sizeof(In));
    // a padding lane's offset lies past every range: it reads zero, stores nothing
    const uint32_t lofs = active ? (uint32_t)((h * D + 8 * c) * sizeof(In)) : 0x80000000u;
    // sequence of t0: [sstart, snext) (packed: the last sequence starting at
    // or before t0, empty sequences skipped)
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
    // uniform across the wave by construction; said so, the row descriptors
    // below stay in scalar registers (else every row load becomes a
    // readfirstlane loop over the descriptor)
    sstart = mx_uniform64(sstart);
    snext = mx_uniform64(snext);
    // the taps first (a small array, mostly from L2): the first row waits only
    // for its own inputs, not for every load of the run
    float taps[K][8];
    const int64_t wofs = active ? (int64_t)h * D + 8 * c : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if constexpr (K == 4) {
            const float4 t4 = reinterpret_cast<const float4*>(Wt)[wofs + i];
            taps[0][i] = t4.x; taps[1][i] = t4.y; taps[2][i] = t4.z; taps[3][i] = t4.w;
        } else {
#pragma unroll
            for (int jj = 0; jj < K; ++jj) taps[jj][i] = Wt[(wofs + i) * K + jj];
        }
    }
    // all loads first.  Inputs: rows from max(sstart, t0 - K + 1) to
    // t0 + nr - 1 (earlier rows fall before the range and read as zero);
    // gates: rows t0 .. t0 + nr - 1.
    const int64_t xr0 = t0 - (K - 1) > sstart ? t0 - (K - 1) : sstart;
    const __amdgpu_buffer_rsrc_t rx = mx_rsrc(x + xr0 * stride, (uint32_t)(t0 + nr - xr0) * rowb);
    const __amdgpu_buffer_rsrc_t rg = mx_rsrc(g + t0 * stride, (uint32_t)nr * rowb);
    Raw8<In> xr[K - 1 + RUN], gr[RUN];
#pragma unroll
    for (int i = 0; i < K - 1 + RUN; ++i)
        ld_raw(rx, (uint32_t)(t0 - (K - 1) + i - xr0) * rowb + lofs, xr[i]);
#pragma unroll
    for (int r = 0; r < RUN; ++r) ld_raw(rg, (uint32_t)r * rowb + lofs, gr[r]);
    const __amdgpu_buffer_rsrc_t ry = mx_rsrc(y + t0 * stride, (uint32_t)nr * rowb);
    const __amdgpu_buffer_rsrc_t rgy = mx_rsrc(gy + t0 * stride, (uint32_t)nr * rowb);
    // row r of the run; `masked`: rows of the run before a sequence start
    // inside it do not feed the rows after it
    auto row = [&](int r, bool masked, int64_t st) {
        const int64_t t = t0 + r;
        float acc[8] = {};
#pragma unroll
        for (int jj = 0; jj < K; ++jj) {
            float xv8[8];
            widen(xr[r + jj], xv8);
            if (masked && t - (K - 1) + jj < st)
#pragma unroll
                for (int i = 0; i < 8; ++i) xv8[i] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(taps[jj][i], xv8[i], acc[i]);
        }
        float yv[8];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            yv[i] = siluf_(acc[i]);
            ss = fmaf(yv[i], yv[i], ss);
        }
        ss = group_sum_dpp<GK>(ss);
        if (j < 2) {
            const float rn = rsqrt_(ss + l2_eps);
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] *= rn;
        }
        float gv[8];
        widen(gr[r], gv);
#pragma unroll
        for (int i = 0; i < 8; ++i) gv[i] = sigmoidf_(gv[i]);
        st_raw(ry, (uint32_t)r * rowb + lofs, yv, y);
        st_raw(rgy, (uint32_t)r * rowb + lofs, gv, gy);
    };
    if (nr == RUN && snext >= t0 + RUN) {
        // a whole run inside one sequence (rows before sstart already read as
        // zero): straight-line rows.  With a branch between rows the
        // compiler's wait at each join covered the previous row's stores too,
        // so every row waited for them to land.
#pragma unroll
        for (int r = 0; r < RUN; ++r) row(r, false, 0);
    } else if (snext >= t0 + nr) {
        // the last, partial run of the rows
#pragma unroll
        for (int r = 0; r < RUN; ++r)
            if (r < nr) row(r, false, 0);
    } else {
        int64_t st = sstart, nx = snext;
#pragma unroll
        for (int r = 0; r < RUN; ++r) {
            if (r >= nr) break;
            const int64_t t = t0 + r;
            if (t == nx) {   // a sequence starts at t: no history
                st = t;
                if (cu) {
                    while (s < nseq - 1 && cu[s + 1] <= t) ++s;
                    nx = cu[s + 1];
                } else {
                    nx = t + T;
                }
            }
            row(r, true, st);
        }
    }
}

// 8 consecutive elements as loaded, with the non-temporal hint: the
// epilogue reads o and the gate once (measured 0.072 against 0.079 ms on the
// 1.3B-layer shape; the same hint on the prologue's gate rows was 1% slower)
__device__ __forceinline__ void ld_raw_nt(const bf16_t* p, Raw8<bf16_t>& x) {
    const mx_u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const mx_u32x4*>(p));
    x.u = make_uint4(u[0], u[1], u[2], u[3]);
}
__device__ __forceinline__ void ld_raw_nt(const float* p, Raw8<float>& x) {
    const floatx4 a = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
    const floatx4 b = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p + 4));
    x.a = make_float4(a[0], a[1], a[2], a[3]);
    x.b = make_float4(b[0], b[1], b[2], b[3]);
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
    // Rows row, row + step and row + 2 step in three register buffers, each
    // loaded two rows ahead of its use and widened only there; rows past the
    // end load the last row (in range, no branch) and are not stored.  A
    // load behind a branch and widened on the spot, or a buffer rotated by
    // copies, waited for that load, and on this hardware the wait (vmcnt)
    // also covered the rows' stores before it.
    auto ld = [&](int64_t r, Raw8<In>& xo, Raw8<In>& go) {
        const int64_t rr = r < nrows ? r : nrows - 1;
        ld_raw_nt(o + (size_t)rr * DV + 8 * c, xo);
        ld_raw_nt(g + (size_t)rr * DV + 8 * c, go);
    };
    auto row_out = [&](int64_t r, const Raw8<In>& xr, const Raw8<In>& gr) {
        float x[8], gg[8];
        widen(xr, x);
        widen(gr, gg);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
        ss = group_sum<G>(ss);
        const float rn = 1.f / sqrtf(ss / DV + eps);
        float out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = x[i] * rn * gm[i] * siluf_(gg[i]);
        st8(y + (size_t)r * DV + 8 * c, out);
    };
    int64_t row = gid / G;
    Raw8<In> x0, g0, x1, g1, x2, g2;
    ld(row, x0, g0);
    ld(row + step, x1, g1);
    for (; row < nrows; row += 3 * step) {
        ld(row + 2 * step, x2, g2);
        row_out(row, x0, g0);
        if (row + step >= nrows) break;
        ld(row + 3 * step, x0, g0);
        row_out(row + step, x1, g1);
        if (row + 2 * step >= nrows) break;
        ld(row + 4 * step, x1, g1);
        row_out(row + 2 * step, x2, g2);
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
    // one thread per (run, lane of the run): every run is covered.  Runs of 8
    // tokens for bf16 (132 registers); fp32 rows take twice
    // the registers, so runs of 4.
    constexpr int RUN = sizeof(In) == 2 ? 8 : 4;
    const int64_t nruns = (rows + RUN - 1) / RUN;
    const int64_t threads = nruns * prologue_short_run_lanes(H, DK, DV);
    // byte offsets inside a run's descriptors are 32-bit
    if ((int64_t)H * (DK > DV ? DK : DV) * (int64_t)sizeof(In) * (RUN + K) >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    if ((threads + MX_THREADS - 1) / MX_THREADS > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((threads + MX_THREADS - 1) / MX_THREADS));
#define GDN2_PRO_ARGS                                                                           \
    static_cast<const In*>(xq), static_cast<const In*>(xk), static_cast<const In*>(xv),         \
        static_cast<const In*>(ga), static_cast<const In*>(gb), static_cast<const In*>(gw), Wq, \
        Wk, Wv, l2_eps, static_cast<In*>(q), static_cast<In*>(k), static_cast<In*>(v),          \
        static_cast<In*>(alpha), static_cast<In*>(b), static_cast<In*>(w), cu, nseq, T, H, rows
    switch (K) {
        case 1: hipLaunchKernelGGL((gdn2_prologue_run_kernel<In, DK, DV, 1, RUN>), grid, dim3(MX_THREADS), 0, stream, GDN2_PRO_ARGS); break;
        case 2: hipLaunchKernelGGL((gdn2_prologue_run_kernel<In, DK, DV, 2, RUN>), grid, dim3(MX_THREADS), 0, stream, GDN2_PRO_ARGS); break;
        case 3: hipLaunchKernelGGL((gdn2_prologue_run_kernel<In, DK, DV, 3, RUN>), grid, dim3(MX_THREADS), 0, stream, GDN2_PRO_ARGS); break;
        default: hipLaunchKernelGGL((gdn2_prologue_run_kernel<In, DK, DV, 4, RUN>), grid, dim3(MX_THREADS), 0, stream, GDN2_PRO_ARGS); break;
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
