// gdn2_decode.hip -- single-token recurrent step (gfx950), and the same step
// walked over whole sequences: the forward for fp32 inputs at dk = 128.
//
// One recurrent step of the Gated Delta Rule-2 per (sequence, head), the
// constant-memory decode the Gated DeltaNet-2 pages credit to linear attention
// (Spanish blog, "Por Que Es Importante" item 1; Korean summary, "results"
// item 2).  The fp32 state is the only large stream: it is read once and
// written once, so the kernel is an HBM read-modify-write.
//
//   S' = Diag(alpha) S                       (decay before the edit)
//   r  = S'^T (b (.) k),  p = S'^T q         (one pass over S')
//   delta = w (.) v - r
//   S <- S' + k delta^T,   o = p + (q . k) delta   (= S_new^T q)
//
// Work split: one workgroup of 256 threads per (sequence, head, 64-column
// value slab); value columns of S are independent.  Thread t owns 4
// consecutive columns (one float4) of 16/8 rows, so a wave reads whole
// 256-byte row segments and every state byte is loaded and stored exactly once.
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

namespace gdn2 {

constexpr int DEC_SLAB = 64;
constexpr int DEC_THREADS = 256;

template <typename In, typename Out, int DK>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const In* __restrict__ alpha, const In* __restrict__ b, const In* __restrict__ w,
    float* __restrict__ S, Out* __restrict__ o, int H, int DV) {
    constexpr int CG = DEC_SLAB / 4;        // threads across a row slab (float4 each)
    constexpr int RG = DEC_THREADS / CG;    // row groups
    constexpr int RPT = DK / RG;            // rows per thread
    const int nslab = DV / DEC_SLAB;
    const int pair = blockIdx.x / nslab;    // n * H + h
    const int slab = blockIdx.x - pair * nslab;
    const int tid = threadIdx.x;
    const int c4 = tid % CG;
    const int rg = tid / CG;
    const int col0 = slab * DEC_SLAB + c4 * 4;

    float* Sp = S + (size_t)pair * DK * DV + col0;
    float4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = *reinterpret_cast<const float4*>(Sp + (size_t)(rg + m * RG) * DV);

    __shared__ float sq[DK], sk[DK], sa[DK], sbk[DK], sx[DEC_SLAB];
    __shared__ float sred[DEC_THREADS / 64][CG][8];
    __shared__ float sqk;
    const size_t kb = (size_t)pair * DK;
    const size_t vb = (size_t)pair * DV + slab * DEC_SLAB;
    if (tid < DK) {
        const float kk = load1(k + kb + tid);
        sq[tid] = load1(q + kb + tid);
        sk[tid] = kk;
        sa[tid] = load1(alpha + kb + tid);
        sbk[tid] = load1(b + kb + tid) * kk;
    }
    if (tid < DEC_SLAB) sx[tid] = load1(w + vb + tid) * load1(v + vb + tid);
    __syncthreads();
    if (tid < 64) {  // q . k by wave 0
        float acc = 0.f;
        for (int i = tid; i < DK; i += 64) acc += sq[i] * sk[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (tid == 0) sqk = acc;
    }

    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const float a = sa[i], bk = sbk[i], qi = sq[i];
        s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
        r0 += bk * s[m].x; r1 += bk * s[m].y; r2 += bk * s[m].z; r3 += bk * s[m].w;
        p0 += qi * s[m].x; p1 += qi * s[m].y; p2 += qi * s[m].z; p3 += qi * s[m].w;
    }
    // sum over the 4 row groups of a wave (lanes c4, c4+16, c4+32, c4+48)
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
        r0 += __shfl_xor(r0, off); r1 += __shfl_xor(r1, off);
        r2 += __shfl_xor(r2, off); r3 += __shfl_xor(r3, off);
        p0 += __shfl_xor(p0, off); p1 += __shfl_xor(p1, off);
        p2 += __shfl_xor(p2, off); p3 += __shfl_xor(p3, off);
    }
    const int wave = tid >> 6;
    if ((tid & 63) < CG) {
        float* d = sred[wave][c4];
        d[0] = r0; d[1] = r1; d[2] = r2; d[3] = r3;
        d[4] = p0; d[5] = p1; d[6] = p2; d[7] = p3;
    }
    __syncthreads();
    float rr[4] = {0.f, 0.f, 0.f, 0.f}, pp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int wv = 0; wv < DEC_THREADS / 64; ++wv)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rr[j] += sred[wv][c4][j];
            pp[j] += sred[wv][c4][4 + j];
        }
    float dl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dl[j] = sx[c4 * 4 + j] - rr[j];

#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const float ki = sk[rg + m * RG];
        float4 t;
        t.x = s[m].x + ki * dl[0]; t.y = s[m].y + ki * dl[1];
        t.z = s[m].z + ki * dl[2]; t.w = s[m].w + ki * dl[3];
        *reinterpret_cast<float4*>(Sp + (size_t)(rg + m * RG) * DV) = t;
    }
    if (rg == 0) {
        const float qk = sqk;
        store4(o + vb + c4 * 4, pp[0] + qk * dl[0], pp[1] + qk * dl[1], pp[2] + qk * dl[2],
               pp[3] + qk * dl[3]);
    }
}

// ---------------------------------------------------------------------------
// token-serial forward, fp32 inputs at dk = 128
// ---------------------------------------------------------------------------
// The same step as decode_kernel, walked over a whole sequence with the state
// slab in registers: S0 is read once, S_T written once, o stored per token.
// This is the forward for fp32 inputs at dk = 128, where the chunked kernel's
// fp32 operand tiles would not fit in LDS; all arithmetic is fp32.
//
// One workgroup per (sequence, head, 64-column slab), thread t owning 4
// columns of DK/16 rows as in decode_kernel.  Tokens go through LDS in blocks
// of SER_TB: while a block is computed, its successor is loaded into
// registers (one float4 of alpha, b, q or k per thread and token, or of w and
// v for the slab) and stored into the other half of a double-buffered stage.
// The partial reads r, p and the partial q . k of a token go through a stage
// double-buffered by token parity.  One barrier per token suffices: a buffer
// is rewritten only after every thread has passed the barrier that follows
// its last read of it.
constexpr int SER_TB = 8;
template <int DK>
__global__ __launch_bounds__(DEC_THREADS) void fwd_serial_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ b, const float* __restrict__ w,
    const float* S0, float* __restrict__ o, float* S_T, const int32_t* __restrict__ cu_seqlens,
    int T, int H, int DV) {
    constexpr int CG = DEC_SLAB / 4;
    constexpr int RG = DEC_THREADS / CG;
    constexpr int RPT = DK / RG;
    constexpr int NW = DEC_THREADS / 64;
    // one token's stage: alpha | b | q | k (DK each) | w (.) v (the slab)
    constexpr int OA = 0, OB = DK, OQ = 2 * DK, OK = 3 * DK, OX = 4 * DK;
    constexpr int STAGE = 4 * DK + DEC_SLAB;
    constexpr int KLOADERS = DK;          // threads loading one key-side float4 per token
    constexpr int XLOADERS = DEC_SLAB / 4;
    static_assert(KLOADERS + XLOADERS <= DEC_THREADS, "loader threads");
    const int nslab = DV / DEC_SLAB;
    const int pair = blockIdx.x / nslab;
    const int slab = blockIdx.x - pair * nslab;
    const int n = pair / H, h = pair - n * H;
    int64_t row0, len;
    if (cu_seqlens) {
        row0 = cu_seqlens[n];
        len = (int64_t)cu_seqlens[n + 1] - row0;
    } else {
        row0 = (int64_t)n * T;
        len = T;
    }
    const int tid = threadIdx.x;
    const int c4 = tid % CG, rg = tid / CG, wave = tid >> 6;
    const int col0 = slab * DEC_SLAB + c4 * 4;
    const size_t sbase = (size_t)pair * DK * DV + col0;

    float4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = S0 ? *reinterpret_cast<const float4*>(S0 + sbase + (size_t)(rg + m * RG) * DV)
                  : make_float4(0.f, 0.f, 0.f, 0.f);

    __shared__ __align__(16) float stage[2][SER_TB][STAGE];
    __shared__ float sred[2][NW][CG][9];
    // loader roles: thread tid < DK loads float4 (tid % (DK/4)) of tensor
    // tid / (DK/4) (alpha, b, q, k); the next DEC_SLAB/4 threads load a float4
    // of w and of v and keep their product
    const int ltensor = tid / (DK / 4), lgrp = tid % (DK / 4);
    const float* lsrc = ltensor == 0 ? alpha : ltensor == 1 ? b : ltensor == 2 ? q : k;
    const int xg = tid - KLOADERS;
    float4 pf[SER_TB];
    auto fetch = [&](int64_t t0) {   // the block of tokens t0 .. t0 + SER_TB - 1 (within len)
#pragma unroll
        for (int u = 0; u < SER_TB; ++u) {
            if (t0 + u >= len) break;
            const size_t tok = (size_t)(row0 + t0 + u) * H + h;
            if (tid < KLOADERS) {
                pf[u] = *reinterpret_cast<const float4*>(lsrc + tok * DK + 4 * lgrp);
            } else if (xg < XLOADERS) {
                const size_t vo = tok * DV + slab * DEC_SLAB + 4 * xg;
                const float4 wv = *reinterpret_cast<const float4*>(w + vo);
                const float4 vv = *reinterpret_cast<const float4*>(v + vo);
                pf[u] = make_float4(wv.x * vv.x, wv.y * vv.y, wv.z * vv.z, wv.w * vv.w);
            }
        }
    };
    auto put = [&](int bufi, int64_t t0) {
#pragma unroll
        for (int u = 0; u < SER_TB; ++u) {
            if (t0 + u >= len) break;
            if (tid < KLOADERS)
                *reinterpret_cast<float4*>(&stage[bufi][u][ltensor * DK + 4 * lgrp]) = pf[u];
            else if (xg < XLOADERS)
                *reinterpret_cast<float4*>(&stage[bufi][u][OX + 4 * xg]) = pf[u];
        }
    };
    if (len > 0) {
        fetch(0);
        put(0, 0);
    }
    __syncthreads();
    for (int64_t t = 0; t < len; ++t) {
        const int u = (int)(t % SER_TB);
        const int blk = (int)((t / SER_TB) & 1);
        const int cur = (int)(t & 1);
        const int64_t tnext = t - u + SER_TB;   // first token of the next block
        if (u == 0 && tnext < len) fetch(tnext);
        const float* st = stage[blk][u];
        float kr[RPT];
        float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f, qk = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + m * RG;
            const float a = st[OA + i], qi = st[OQ + i];
            kr[m] = st[OK + i];
            const float bk = st[OB + i] * kr[m];
            s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
            r0 += bk * s[m].x; r1 += bk * s[m].y; r2 += bk * s[m].z; r3 += bk * s[m].w;
            p0 += qi * s[m].x; p1 += qi * s[m].y; p2 += qi * s[m].z; p3 += qi * s[m].w;
            qk += qi * kr[m];
        }
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = st[OX + c4 * 4 + j];
        // sum over the 4 row groups of a wave (lanes c4, c4+16, c4+32, c4+48)
#pragma unroll
        for (int off = CG; off < 64; off <<= 1) {
            r0 += __shfl_xor(r0, off); r1 += __shfl_xor(r1, off);
            r2 += __shfl_xor(r2, off); r3 += __shfl_xor(r3, off);
            p0 += __shfl_xor(p0, off); p1 += __shfl_xor(p1, off);
            p2 += __shfl_xor(p2, off); p3 += __shfl_xor(p3, off);
            qk += __shfl_xor(qk, off);
        }
        if ((tid & 63) < CG) {
            float* d = sred[cur][wave][c4];
            d[0] = r0; d[1] = r1; d[2] = r2; d[3] = r3;
            d[4] = p0; d[5] = p1; d[6] = p2; d[7] = p3;
            d[8] = qk;
        }
        if (u == SER_TB - 1 && tnext < len) put(blk ^ 1, tnext);
        __syncthreads();
        float rr[4] = {0.f, 0.f, 0.f, 0.f}, pp[4] = {0.f, 0.f, 0.f, 0.f};
        float qkt = 0.f;   // q . k over all rows: each wave's column-group-0 sum
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                rr[j] += sred[cur][wv][c4][j];
                pp[j] += sred[cur][wv][c4][4 + j];
            }
            qkt += sred[cur][wv][0][8];
        }
        float dl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) dl[j] = x[j] - rr[j];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            s[m].x += kr[m] * dl[0]; s[m].y += kr[m] * dl[1];
            s[m].z += kr[m] * dl[2]; s[m].w += kr[m] * dl[3];
        }
        if (rg == 0)
            store4(o + ((size_t)(row0 + t) * H + h) * DV + col0, pp[0] + qkt * dl[0],
                   pp[1] + qkt * dl[1], pp[2] + qkt * dl[2], pp[3] + qkt * dl[3]);
    }
    if (S_T) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            *reinterpret_cast<float4*>(S_T + sbase + (size_t)(rg + m * RG) * DV) = s[m];
    }
}

hipError_t launch_fwd_serial(const float* q, const float* k, const float* v, const float* alpha,
                             const float* b, const float* w, const float* S0, float* o,
                             float* S_T, const int32_t* cu_seqlens, int N, int T, int H, int dk,
                             int dv, hipStream_t stream) {
    const dim3 grid((unsigned)((size_t)N * H * (dv / DEC_SLAB)));
    const dim3 block(DEC_THREADS);
    if (dk == 128)
        hipLaunchKernelGGL((fwd_serial_kernel<128>), grid, block, 0, stream, q, k, v, alpha, b, w,
                           S0, o, S_T, cu_seqlens, T, H, dv);
    else
        hipLaunchKernelGGL((fwd_serial_kernel<64>), grid, block, 0, stream, q, k, v, alpha, b, w,
                           S0, o, S_T, cu_seqlens, T, H, dv);
    return hipGetLastError();
}

template <typename In, typename Out>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const void* alpha,
                                  const void* b, const void* w, float* S, void* o, int N, int H,
                                  int dk, int dv, hipStream_t stream) {
    const dim3 grid((unsigned)((size_t)N * H * (dv / DEC_SLAB)));
    const dim3 block(DEC_THREADS);
#define GDN2_DEC_ARGS                                                                       \
    static_cast<const In*>(q), static_cast<const In*>(k), static_cast<const In*>(v),       \
        static_cast<const In*>(alpha), static_cast<const In*>(b), static_cast<const In*>(w), \
        S, static_cast<Out*>(o), H, dv
    if (dk == 128)
        hipLaunchKernelGGL((decode_kernel<In, Out, 128>), grid, block, 0, stream, GDN2_DEC_ARGS);
    else
        hipLaunchKernelGGL((decode_kernel<In, Out, 64>), grid, block, 0, stream, GDN2_DEC_ARGS);
#undef GDN2_DEC_ARGS
    return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* alpha,
                         const void* b, const void* w, int in_dtype, float* S, void* o,
                         int out_dtype, int N, int H, int dk, int dv, hipStream_t stream) {
    if (in_dtype == DT_BF16) {
        if (out_dtype == DT_BF16)
            return launch_decode_t<bf16_t, bf16_t>(q, k, v, alpha, b, w, S, o, N, H, dk, dv, stream);
        return launch_decode_t<bf16_t, float>(q, k, v, alpha, b, w, S, o, N, H, dk, dv, stream);
    }
    return launch_decode_t<float, float>(q, k, v, alpha, b, w, S, o, N, H, dk, dv, stream);
}

}  // namespace gdn2
