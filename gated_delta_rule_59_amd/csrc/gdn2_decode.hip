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
// Work split: one workgroup of 256 threads per (sequence, head, 32-column
// value slab); value columns of S are independent.  Thread t owns 4
// consecutive columns (one float4) of 4 (dk = 128) or 2 rows, so eight lanes
// cover one 128-byte row segment and every state byte is loaded and stored
// exactly once.  (64-column slabs with 8 rows per thread measured 3% slower,
// 16-column slabs with 64-byte segments 50% slower.)
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

namespace gdn2 {

constexpr int DEC_SLAB = 32;
constexpr int DEC_THREADS = 256;

template <typename In, typename Out, int DK>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const In* __restrict__ alpha, const In* __restrict__ b, const In* __restrict__ w,
    float* __restrict__ S, Out* __restrict__ o, int H, int DV, int gates) {
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
        // a per-(token, head) gate ([N, H]) is broadcast over the channels
        sa[tid] = load1(alpha + (gates == GATES_GDN ? (size_t)pair : kb + tid));
        sbk[tid] = load1(b + (gates != GATES_FULL ? (size_t)pair : kb + tid)) * kk;
    }
    if (tid < DEC_SLAB)
        sx[tid] = load1(w + (gates != GATES_FULL ? (size_t)pair : vb + tid)) * load1(v + vb + tid);
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
// The decode step walked over a whole sequence with the state in registers:
// S0 is read once, S_T written once, o stored per token.  This is the forward
// for fp32 inputs at dk = 128, where the chunked kernel's fp32 operand tiles
// would not fit in LDS; all arithmetic is fp32.
//
// One wave per (sequence, head, 16 value columns); lane l owns key rows
// l*RPL .. l*RPL+RPL-1 (RPL = DK/64) of those 16 columns.  The column sums
// r = S'^T (b (.) k) and p = S'^T q over all DK rows are reduce-scattered
// across the wave with lane swaps only (v_permlane32_swap, v_permlane16_swap,
// DPP mirrors and quad permutes): afterwards lane l holds column l >> 2.
// delta is then gathered back to every lane the same way.  No LDS and no
// barrier; the next SER_PF tokens' inputs are loaded while a token is
// computed.
constexpr int SER_PF = 4;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_ROW_MIRROR = 0x140, DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_QP_XOR2 = 0x4E /* quad_perm [2,3,0,1] */, DPP_QP_XOR1 = 0xB1 /* [1,0,3,2] */;
constexpr int DPP_ROW_ROR8 = 0x128, DPP_ROW_ROR4 = 0x124, DPP_ROW_ROR2 = 0x122,
              DPP_ROW_ROR1 = 0x121;

// v[16] (columns 0..15, a partial sum per lane) -> the full sum over the 64
// lanes of column l >> 2, in every lane
__device__ __forceinline__ float reduce_scatter16(const float (&v)[16], int l) {
    float u[8], w[4];
#pragma unroll
    for (int m = 0; m < 8; ++m) u[m] = swap32_sum(v[m], v[m + 8]);   // column m + 8 b5
#pragma unroll
    for (int m = 0; m < 4; ++m) w[m] = swap16_sum(u[m], u[m + 4]);          // + 4 b4
    const bool b3 = (l >> 3) & 1, b2 = (l >> 2) & 1;
    // pair l <-> 15 - l (bit 3 differs): keep columns {0,1} or {2,3} of w
    const float k0 = b3 ? w[2] : w[0], k1 = b3 ? w[3] : w[1];
    const float s0 = b3 ? w[0] : w[2], s1 = b3 ? w[1] : w[3];
    const float z0 = k0 + dpp<DPP_ROW_MIRROR>(s0), z1 = k1 + dpp<DPP_ROW_MIRROR>(s1);
    // pair l <-> 7 - l within 8 lanes (bit 2 differs): keep column 0 or 1
    const float kk = b2 ? z1 : z0, ss = b2 ? z0 : z1;
    float y = kk + dpp<DPP_ROW_HALF_MIRROR>(ss);
    y += dpp<DPP_QP_XOR2>(y);   // the four lanes l & ~3 .. +3 share the column
    y += dpp<DPP_QP_XOR1>(y);
    return y;
}
// a scalar summed over the 64 lanes, in every lane
__device__ __forceinline__ float reduce_all(float x) {
    x = swap32_sum(x, x);
    x = swap16_sum(x, x);
    x += dpp<DPP_ROW_ROR8>(x);
    x += dpp<DPP_ROW_ROR4>(x);
    x += dpp<DPP_ROW_ROR2>(x);
    x += dpp<DPP_ROW_ROR1>(x);
    return x;
}
// lane l holds column l >> 2 (the same value in lanes l & ~3 .. +3) -> all
// 16 columns in every lane
__device__ __forceinline__ void all_gather16(float d, int l, float (&out)[16]) {
    const bool b3 = (l >> 3) & 1, b2 = (l >> 2) & 1;
    // columns 2 c + {0, 1}, c = l >> 3: the partner l <-> 7 - l holds the other
    const float pd = dpp<DPP_ROW_HALF_MIRROR>(d);
    const float e0 = b2 ? pd : d, e1 = b2 ? d : pd;
    // columns 4 (l >> 4) + {0..3}: the partner l <-> 15 - l holds the other pair
    const float p0 = dpp<DPP_ROW_MIRROR>(e0), p1 = dpp<DPP_ROW_MIRROR>(e1);
    float f[4];
    f[0] = b3 ? p0 : e0; f[1] = b3 ? p1 : e1; f[2] = b3 ? e0 : p0; f[3] = b3 ? e1 : p1;
    float g8[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {   // rows 0,2 hold columns m, rows 1,3 columns m + 4
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(f[m]), __float_as_uint(f[m]),
                                                        false, false);
        g8[m] = __uint_as_float(r[0]);
        g8[m + 4] = __uint_as_float(r[1]);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {   // lanes 0..31 hold columns m, lanes 32..63 columns m + 8
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(g8[m]), __float_as_uint(g8[m]),
                                                        false, false);
        out[m] = __uint_as_float(r[0]);
        out[m + 8] = __uint_as_float(r[1]);
    }
}

template <int DK>
__global__ __launch_bounds__(64) void fwd_serial_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ b, const float* __restrict__ w,
    const float* S0, float* __restrict__ o, float* S_T, const int32_t* __restrict__ cu_seqlens,
    int T, int H, int DV, int gates) {
    constexpr int RPL = DK / 64;   // key rows per lane
    const int ncb = DV / 16;
    const int pair = blockIdx.x / ncb;
    const int c0 = (blockIdx.x - pair * ncb) * 16;
    const int n = pair / H, h = pair - n * H;
    int64_t row0, len;
    if (cu_seqlens) {
        row0 = cu_seqlens[n];
        len = (int64_t)cu_seqlens[n + 1] - row0;
    } else {
        row0 = (int64_t)n * T;
        len = T;
    }
    const int l = threadIdx.x;
    const int cf = l >> 2;   // the column this lane holds after the reduce-scatter
    const size_t sbase = (size_t)pair * DK * DV + c0;

    float s[RPL][16];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const float* src = S0 ? S0 + sbase + (size_t)(l * RPL + i) * DV : nullptr;
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
            const float4 x = src ? *reinterpret_cast<const float4*>(src + j) : make_float4(0.f, 0.f, 0.f, 0.f);
            s[i][j] = x.x; s[i][j + 1] = x.y; s[i][j + 2] = x.z; s[i][j + 3] = x.w;
        }
    }

    // the inputs of one token for this lane: its key rows of alpha, b, q, k
    // and w, v of column c0 + cf
    struct Tok { float a[RPL], bb[RPL], qq[RPL], kk[RPL], ww, vv; };
    auto fetch = [&](int64_t t, Tok& x) {
        if (t >= len) return;
        const size_t kr = ((size_t)(row0 + t) * H + h) * DK + (size_t)l * RPL;
        const size_t vr = ((size_t)(row0 + t) * H + h) * DV + c0 + cf;
        const size_t th = (size_t)(row0 + t) * H + h;   // a per-(token, head) gate
        const bool ga = gates == GATES_GDN, gbw = gates != GATES_FULL;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            x.a[i] = alpha[ga ? th : kr + i];
            x.bb[i] = b[gbw ? th : kr + i];
            x.qq[i] = q[kr + i];
            x.kk[i] = k[kr + i];
        }
        x.ww = w[gbw ? th : vr];
        x.vv = v[vr];
    };
    Tok pf[SER_PF];
#pragma unroll
    for (int u = 0; u < SER_PF; ++u) fetch(u, pf[u]);

    for (int64_t t0 = 0; t0 < len; t0 += SER_PF) {
#pragma unroll
        for (int u = 0; u < SER_PF; ++u) {
            const int64_t t = t0 + u;
            if (t >= len) break;
            const Tok x = pf[u];
            fetch(t + SER_PF, pf[u]);
            float r[16], p[16], qk = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) { r[j] = 0.f; p[j] = 0.f; }
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const float bk = x.bb[i] * x.kk[i];
                qk += x.qq[i] * x.kk[i];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    s[i][j] *= x.a[i];
                    r[j] += bk * s[i][j];
                    p[j] += x.qq[i] * s[i][j];
                }
            }
            const float rf = reduce_scatter16(r, l), pfc = reduce_scatter16(p, l);
            const float qkt = reduce_all(qk);
            const float d = x.ww * x.vv - rf;   // delta of column cf
            if ((l & 3) == 0) o[((size_t)(row0 + t) * H + h) * DV + c0 + cf] = pfc + qkt * d;
            float dl[16];
            all_gather16(d, l, dl);
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) s[i][j] += x.kk[i] * dl[j];
        }
    }
    if (S_T) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            float* dst = S_T + sbase + (size_t)(l * RPL + i) * DV;
#pragma unroll
            for (int j = 0; j < 16; j += 4)
                *reinterpret_cast<float4*>(dst + j) = make_float4(s[i][j], s[i][j + 1], s[i][j + 2], s[i][j + 3]);
        }
    }
}

hipError_t launch_fwd_serial(const float* q, const float* k, const float* v, const float* alpha,
                             const float* b, const float* w, const float* S0, float* o,
                             float* S_T, const int32_t* cu_seqlens, int N, int T, int H, int dk,
                             int dv, int gates, hipStream_t stream) {
    const dim3 grid((unsigned)((size_t)N * H * (dv / 16)));
    const dim3 block(64);
    if (dk == 128)
        hipLaunchKernelGGL((fwd_serial_kernel<128>), grid, block, 0, stream, q, k, v, alpha, b, w,
                           S0, o, S_T, cu_seqlens, T, H, dv, gates);
    else
        hipLaunchKernelGGL((fwd_serial_kernel<64>), grid, block, 0, stream, q, k, v, alpha, b, w,
                           S0, o, S_T, cu_seqlens, T, H, dv, gates);
    return hipGetLastError();
}

template <typename In, typename Out>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const void* alpha,
                                  const void* b, const void* w, float* S, void* o, int N, int H,
                                  int dk, int dv, int gates, hipStream_t stream) {
    const dim3 grid((unsigned)((size_t)N * H * (dv / DEC_SLAB)));
    const dim3 block(DEC_THREADS);
#define GDN2_DEC_ARGS                                                                       \
    static_cast<const In*>(q), static_cast<const In*>(k), static_cast<const In*>(v),       \
        static_cast<const In*>(alpha), static_cast<const In*>(b), static_cast<const In*>(w), \
        S, static_cast<Out*>(o), H, dv, gates
    if (dk == 128)
        hipLaunchKernelGGL((decode_kernel<In, Out, 128>), grid, block, 0, stream, GDN2_DEC_ARGS);
    else
        hipLaunchKernelGGL((decode_kernel<In, Out, 64>), grid, block, 0, stream, GDN2_DEC_ARGS);
#undef GDN2_DEC_ARGS
    return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* alpha,
                         const void* b, const void* w, int in_dtype, float* S, void* o,
                         int out_dtype, int N, int H, int dk, int dv, int gates,
                         hipStream_t stream) {
    if (in_dtype == DT_BF16) {
        if (out_dtype == DT_BF16)
            return launch_decode_t<bf16_t, bf16_t>(q, k, v, alpha, b, w, S, o, N, H, dk, dv, gates, stream);
        return launch_decode_t<bf16_t, float>(q, k, v, alpha, b, w, S, o, N, H, dk, dv, gates, stream);
    }
    return launch_decode_t<float, float>(q, k, v, alpha, b, w, S, o, N, H, dk, dv, gates, stream);
}

}  // namespace gdn2
