// gdn2_bwd.hip -- gate-aware chunked backward of the Gated Delta Rule-2
// (gfx950).
//
// The pages name a backward that keeps the gradient flowing through both the
// erase gate b and the write gate w without extra memory beyond the chunk
// states (Spanish blog "Innovaciones Tecnicas" item 2; Korean summary,
// "method", closing paragraph).  This file differentiates the chunk algebra
// of the forward.  With chunk start state S, midpoint row m = 31, the
// in-chunk decay factor e1_r = gamma_r / gamma_mid per key channel,
// Gm = gamma_mid and GR = gamma_C / gamma_mid:
//
//   Kt'_r = b_r k_r e1_r    Qt'_r = q_r e1_r    Kh'_r = k_r / e1_r    X_r = w_r v_r
//   A = strictly_lower(Kt' Kh'^T)   P = tril(Qt' Kh'^T)   T = (I + A)^-1
//   Sm = Gm S   Delta = T (X - Kt' Sm)   O = Qt' Sm + P Delta
//   S_next = GR (Sm + Kh'^T Delta)
//
// and, for the loss sum <dO, O> + <dS_T, S_T>, given dN = dL/dS_next:
//
//   dU = GR dN                dDelta = P^T dO + Kh' dU      dZ = T^T dDelta
//   dSm = Qt'^T dO + dU - Kt'^T dZ                          dS = Gm dSm
//   dX = dZ  (dw = dZ v, dv = dZ w)
//   dP = tril(dO Delta^T)     dA = -strictly_lower(dZ Delta^T)
//   dQt' = dO Sm^T + dP Kh'   dKt' = -dZ Sm^T + dA Kh'
//   dKh' = dP^T Qt' + dA^T Kt' + Delta dU^T
//   dq = dQt' e1   db = dKt' k e1   dk = dKt' b e1 + dKh' / e1
//
// The decay enters only through ln gamma: with e_r = dKt'_r Kt'_r + dQt'_r
// Qt'_r - dKh'_r Kh'_r (per channel), cS = rowsum(dSm Sm), cC =
// rowsum(dN S_next), the gradient of ln alpha_s is
//   sum_{r >= s} e_r + [s <= m] (cS - cC - sum_r e_r) + cC,
// and dalpha = that / alpha.
//
// Kernels (all arithmetic fp32; the forward runs first in its checkpoint
// mode, storing every chunk's start state):
//   bwd_slots_kernel  slot offsets of the sequences' chunks (packed batches)
//   bwd_prep_kernel   per (chunk, head): the tiles Kt', Qt', Kh', A, P,
//                     T = (I + A)^-1 (16x16 diagonal blocks by substitution,
//                     the rest by block products), Delta, and Gm, GR
//   bwd_dstate_kernel per (sequence, head, 32 value columns), 8 waves: the
//                     reverse walk over chunks carrying dL/dS; stores dU and
//                     dZ per chunk, writes dv, dw and dS0, and the row sums
//                     cS, cC.  The column slabs of one (sequence, head) run
//                     on one XCD, so they share the chunk's tiles in its L2.
//   bwd_grad_kernel   per (chunk, head), 8 waves: the products over the value
//                     axis and the chunk axis above, then dq, dk, db, dalpha
// Every operand block is staged into LDS with all of a thread's loads issued
// before its stores; the inner loops read LDS only.
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

constexpr int BC = 64;        // chunk length
constexpr int BMID = 31;      // midpoint row of a chunk
constexpr int BT = 256;       // threads per workgroup (prep, grad)
constexpr int BT2 = 512;      // threads per workgroup (reverse walk)
constexpr int BSV = 32;       // value columns per reverse-walk workgroup

struct BwdArgs {
    const void *q, *k, *v, *alpha, *b, *w, *dout;
    const float* S0;       // [N, H, dk, dv] or null
    const float* dS_T;     // [N, H, dk, dv] or null
    void *dq, *dk, *dv, *dalpha, *db, *dw;
    float* dS0;            // [N, H, dk, dv] or null
    const int32_t* cu;     // packed offsets or null
    int N, T, H;
    const int64_t* coff;   // [N + 1] first slot of each sequence (ckpt_slot0), total at N
    // per (slot, head) buffers
    const float* ck;       // [slot][H][dk][dv]  chunk start states (ckpt_slot0 layout)
    float *kt, *qt, *kh;   // [slot][H][C][dk]   Kt', Qt', Kh'
    float* pm;             // [slot][H][C][C]    P
    float* tm;             // [slot][H][C][C]    T
    float* dl;             // [slot][H][C][dv]   Delta
    float* gr;             // [slot][H][2][dk]   Gm, GR
    float* du;             // [slot][H][dk][dv]  dU
    float* dz;             // [slot][H][C][dv]   dZ
    float* cf;             // [slot][H][nsl][2][dk]  cS, cC partial row sums per column slab
    int nsl;               // value-column slabs of the reverse walk
};

__device__ __forceinline__ float ldf(const bf16_t* p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ float ldf(const float* p) { return *p; }
__device__ __forceinline__ float4 ld4f(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4f(const bf16_t* p) {
    const u16x4 u = *reinterpret_cast<const u16x4*>(p);
    return make_float4(bf16_to_f32(u[0]), bf16_to_f32(u[1]), bf16_to_f32(u[2]), bf16_to_f32(u[3]));
}
__device__ __forceinline__ float4 zf4() { return make_float4(0.f, 0.f, 0.f, 0.f); }
__device__ __forceinline__ void st4s(float* d, float4 x) {   // LDS, any pitch
    d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
}

// Stages rows 0 .. ROWS-1, columns 0 .. COLS-1 of a row-major block (row
// stride `stride` elements) into LDS with pitch PITCH, times `scale` per
// row when given; rows >= valid read as zero.  A thread issues all of its
// loads before its first store.
template <int ROWS, int COLS, int PITCH, int NTH, typename Src>
__device__ __forceinline__ void stage(float* dst, const Src* src, size_t stride, int valid,
                                      const float* rowscale = nullptr) {
    constexpr int C4 = COLS / 4, N4 = ROWS * C4, PER = (N4 + NTH - 1) / NTH;
    const int t = threadIdx.x;
    float4 buf[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = t + u * NTH;
        const int r = e / C4, c = e - r * C4;
        buf[u] = (e < N4 && r < valid) ? ld4f(src + (size_t)r * stride + 4 * c) : zf4();
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = t + u * NTH;
        if (e < N4) {
            const int r = e / C4, c = e - r * C4;
            float4 x = buf[u];
            if (rowscale) {
                const float sc = rowscale[r];
                x.x *= sc; x.y *= sc; x.z *= sc; x.w *= sc;
            }
            st4s(dst + r * PITCH + 4 * c, x);
        }
    }
}

// As stage, transposed: element (r, c) of the block lands at dst[c * PITCH + r].
template <int ROWS, int COLS, int PITCH, int NTH, typename Src>
__device__ __forceinline__ void stage_t(float* dst, const Src* src, size_t stride, int valid,
                                        const float* rowscale = nullptr) {
    constexpr int C4 = COLS / 4, N4 = ROWS * C4, PER = (N4 + NTH - 1) / NTH;
    const int t = threadIdx.x;
    float4 buf[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = t + u * NTH;
        const int r = e / C4, c = e - r * C4;
        buf[u] = (e < N4 && r < valid) ? ld4f(src + (size_t)r * stride + 4 * c) : zf4();
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = t + u * NTH;
        if (e < N4) {
            const int r = e / C4, c = e - r * C4;
            const float sc = rowscale ? rowscale[r] : 1.f;
            dst[(4 * c + 0) * PITCH + r] = buf[u].x * sc;
            dst[(4 * c + 1) * PITCH + r] = buf[u].y * sc;
            dst[(4 * c + 2) * PITCH + r] = buf[u].z * sc;
            dst[(4 * c + 3) * PITCH + r] = buf[u].w * sc;
        }
    }
}

// Sequence n: first token row and length.
__device__ __forceinline__ void seq_of(const BwdArgs& a, int n, int64_t& row0, int64_t& len) {
    if (a.cu) {
        row0 = a.cu[n];
        len = (int64_t)a.cu[n + 1] - row0;
    } else {
        row0 = (int64_t)n * a.T;
        len = a.T;
    }
}

// The (sequence, chunk) of slot g, or false for a final-state slot or a slot
// past the end.
__device__ __forceinline__ bool chunk_of_slot(const BwdArgs& a, int64_t g, int& n, int64_t& c) {
    if (g >= a.coff[a.N]) return false;
    int lo = 0, hi = a.N - 1;   // largest n with coff[n] <= g
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.coff[mid] <= g) lo = mid;
        else hi = mid - 1;
    }
    n = lo;
    c = g - a.coff[n];
    int64_t row0, len;
    seq_of(a, n, row0, len);
    return c < (len + BC - 1) / BC;
}

// In-chunk decay factors of one chunk: e1[r][i] = gamma_r / gamma_mid (rows
// past the chunk's end count as alpha = 1), gm[i] = gamma_mid, gR[i] =
// gamma_C / gamma_mid.  One thread per key channel walks the rows from the
// midpoint outwards, so no factor carries more than half a chunk of decay.
template <typename In, int DK, int PE>
__device__ __forceinline__ void chunk_factors(const In* alpha, size_t base, size_t rstride, int clen,
                                              float* sE, float* gm, float* gR) {
    const int i = threadIdx.x;
    if (i >= DK) return;
    float al[BC];
#pragma unroll
    for (int r = 0; r < BC; ++r) al[r] = r < clen ? ldf(alpha + base + (size_t)r * rstride + i) : 1.f;
    float p = 1.f;   // product over rows (r, mid]
#pragma unroll
    for (int r = BMID; r >= 0; --r) {
        sE[r * PE + i] = 1.f / p;
        p *= al[r];
    }
    float qv = 1.f;  // product over rows (mid, r]
#pragma unroll
    for (int r = BMID + 1; r < BC; ++r) {
        qv *= al[r];
        sE[r * PE + i] = qv;
    }
    gm[i] = p;
    gR[i] = qv;
}

}  // namespace

// ---------------------------------------------------------------------------
// slot offsets: coff[n] = ckpt_slot0(n), coff[N] = total slots
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BT) void bwd_slots_kernel(const int32_t* __restrict__ cu, int N, int T,
                                                       int64_t* __restrict__ coff) {
    __shared__ int64_t part[BT];
    const int t = threadIdx.x;
    if (!cu) {
        for (int n = t; n <= N; n += BT) coff[n] = (int64_t)n * ((T + BC - 1) / BC + 1);
        return;
    }
    // each thread sums a contiguous block of sequences, then an exclusive
    // scan of the block sums
    const int per = (N + BT - 1) / BT;
    const int n0 = t * per, n1 = min(N, n0 + per);
    int64_t s = 0;
    for (int n = n0; n < n1; ++n) s += ((int64_t)cu[n + 1] - cu[n] + BC - 1) / BC + 1;
    part[t] = s;
    __syncthreads();
    if (t == 0) {
        int64_t acc = 0;
        for (int u = 0; u < BT; ++u) {
            const int64_t x = part[u];
            part[u] = acc;
            acc += x;
        }
    }
    __syncthreads();
    int64_t acc = part[t];
    for (int n = n0; n < n1; ++n) {
        coff[n] = acc;
        acc += ((int64_t)cu[n + 1] - cu[n] + BC - 1) / BC + 1;
    }
    if (t == BT - 1) coff[N] = acc;
}

// ---------------------------------------------------------------------------
// per (chunk, head): tiles, A, P, T = (I + A)^-1, Delta, Gm, GR
// ---------------------------------------------------------------------------
template <typename In, int DK, int DV>
__global__ __launch_bounds__(BT) void bwd_prep_kernel(BwdArgs a) {
    constexpr int PE = DK + 1;   // pitch of the [C][DK] tiles
    constexpr int PA = BC + 1;   // pitch of the [C][C] tiles
    constexpr int PZ = DV + 1;   // pitch of Z
    constexpr int PSL = BSV + 1;
    __shared__ float sE[BC * PE];                      // e1, then Kt'
    __shared__ float sQ[BC * PE];                      // Qt'
    __shared__ float sKH[BC * (PE > PZ ? PE : PZ)];   // Kh', then Z = X - Kt' Sm
    __shared__ float sA[BC * PA];
    __shared__ float sT[BC * PA];
    __shared__ float sS[DK * PSL];                     // a 32-column slice of Sm
    __shared__ float sgm[DK], sgr[DK];

    const int h = blockIdx.y;
    const int64_t g = blockIdx.x;
    int n;
    int64_t c;
    if (!chunk_of_slot(a, g, n, c)) return;
    const int H = a.H, t = threadIdx.x;
    int64_t row0, len;
    seq_of(a, n, row0, len);
    const int clen = (int)min((int64_t)BC, len - c * BC);
    const size_t kst = (size_t)H * DK, vst = (size_t)H * DV;
    const size_t kb = ((size_t)(row0 + c * BC) * H + h) * DK;   // row 0 of the chunk, head h
    const size_t vb = ((size_t)(row0 + c * BC) * H + h) * DV;
    const In* q = static_cast<const In*>(a.q);
    const In* k = static_cast<const In*>(a.k);
    const In* v = static_cast<const In*>(a.v);
    const In* b = static_cast<const In*>(a.b);
    const In* w = static_cast<const In*>(a.w);
    const size_t gh = (size_t)g * H + h;

    chunk_factors<In, DK, PE>(static_cast<const In*>(a.alpha), kb, kst, clen, sE, sgm, sgr);
    __syncthreads();
    if (t < DK) {
        a.gr[gh * 2 * DK + t] = sgm[t];
        a.gr[gh * 2 * DK + DK + t] = sgr[t];
    }
    // tiles over e1, four channels at a time: Kh' = k / e1, Kt' = b k e1,
    // Qt' = q e1, into LDS and the workspace
    {
        constexpr int C4 = DK / 4, PER = BC * C4 / BT;
        float4 kk[PER], bb[PER], qq[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = t + u * BT, r = e / C4, c4 = e - r * C4;
            const size_t o = kb + (size_t)r * kst + 4 * c4;
            const bool ok = r < clen;
            kk[u] = ok ? ld4f(k + o) : zf4();
            bb[u] = ok ? ld4f(b + o) : zf4();
            qq[u] = ok ? ld4f(q + o) : zf4();
        }
        float* gkt = a.kt + gh * BC * DK;
        float* gqt = a.qt + gh * BC * DK;
        float* gkh = a.kh + gh * BC * DK;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = t + u * BT, r = e / C4, c4 = e - r * C4;
            float* pe = sE + r * PE + 4 * c4;
            const float e1[4] = {pe[0], pe[1], pe[2], pe[3]};
            const float xk[4] = {kk[u].x, kk[u].y, kk[u].z, kk[u].w};
            const float xb[4] = {bb[u].x, bb[u].y, bb[u].z, bb[u].w};
            const float xq[4] = {qq[u].x, qq[u].y, qq[u].z, qq[u].w};
            float vkt[4], vqt[4], vkh[4];
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                vkh[z] = xk[z] / e1[z];
                vkt[z] = xb[z] * xk[z] * e1[z];
                vqt[z] = xq[z] * e1[z];
                pe[z] = vkt[z];
                sQ[r * PE + 4 * c4 + z] = vqt[z];
                sKH[r * PE + 4 * c4 + z] = vkh[z];
            }
            const size_t go = (size_t)r * DK + 4 * c4;
            *reinterpret_cast<float4*>(gkt + go) = make_float4(vkt[0], vkt[1], vkt[2], vkt[3]);
            *reinterpret_cast<float4*>(gqt + go) = make_float4(vqt[0], vqt[1], vqt[2], vqt[3]);
            *reinterpret_cast<float4*>(gkh + go) = make_float4(vkh[0], vkh[1], vkh[2], vkh[3]);
        }
    }
    __syncthreads();
    // A = strictly_lower(Kt' Kh'^T) and P = tril(Qt' Kh'^T): thread (rows
    // 4 tr.., cols 4 tc..)
    {
        const int tr = t >> 4, tc = t & 15;
        float acc[4][4] = {}, pcc[4][4] = {};
        for (int i = 0; i < DK; ++i) {
            float x[4], y[4], z4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[u] = sE[(4 * tr + u) * PE + i];
                z4[u] = sQ[(4 * tr + u) * PE + i];
                y[u] = sKH[(4 * tc + u) * PE + i];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    acc[u][z] += x[u] * y[z];
                    pcc[u][z] += z4[u] * y[z];
                }
        }
        float* P = a.pm + gh * BC * BC;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 4 * tr + u;
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int s2 = 4 * tc + z;
                sA[r * PA + s2] = s2 < r ? acc[u][z] : 0.f;
                sT[r * PA + s2] = 0.f;
            }
            *reinterpret_cast<float4*>(P + r * BC + 4 * tc) =
                make_float4(4 * tc <= r ? pcc[u][0] : 0.f, 4 * tc + 1 <= r ? pcc[u][1] : 0.f,
                            4 * tc + 2 <= r ? pcc[u][2] : 0.f, 4 * tc + 3 <= r ? pcc[u][3] : 0.f);
        }
    }
    // Z = X - Kt' Sm, by 32-column slices of Sm = Gm (.) S staged in LDS:
    // thread (row zr, 8 columns zc.. of each slice)
    constexpr int NSL = DV / BSV;
    const int zr = t >> 2, zc = (t & 3) * 8;
    float Z[NSL][8];
    const float* S = a.ck + gh * DK * DV;
    for (int sl = 0; sl < NSL; ++sl) {
        __syncthreads();   // the previous slice (and, first time, the tiles) is done
        stage<DK, BSV, PSL, BT>(sS, S + sl * BSV, DV, DK, sgm);
        __syncthreads();
        float acc[8] = {};
        for (int i = 0; i < DK; ++i) {
            const float x = sE[zr * PE + i];
#pragma unroll
            for (int z = 0; z < 8; ++z) acc[z] += x * sS[i * PSL + zc + z];
        }
#pragma unroll
        for (int z = 0; z < 8; ++z) {
            float xv = 0.f;
            if (zr < clen) {
                const size_t o = vb + (size_t)zr * vst + sl * BSV + zc + z;
                xv = ldf(w + o) * ldf(v + o);
            }
            Z[sl][z] = xv - acc[z];
        }
    }
    // T = (I + A)^-1: the four 16x16 diagonal blocks by forward substitution
    // (one column per thread), then block row i from the rows above it:
    // T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj
    __syncthreads();
    if (t < BC) {
        const int bi = t >> 4, j = t & 15, o = 16 * bi;
        for (int r = 0; r < 16; ++r) {
            float x = r == j ? 1.f : 0.f;
            for (int s2 = j; s2 < r; ++s2) x -= sA[(o + r) * PA + o + s2] * sT[(o + s2) * PA + o + j];
            sT[(o + r) * PA + o + j] = x;
        }
    }
    for (int bi = 1; bi < 4; ++bi) {
        __syncthreads();
        // X_ij = sum_{m=j}^{bi-1} A_im T_mj for j < bi, into the T_ij places
        float xr[3];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            xr[u] = 0.f;
            const int e = t + u * BT;   // element of the bi x 256 block row
            if (u < bi) {
                const int j = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
                const int r = 16 * bi + rr, col = 16 * j + cc;
                float x = 0.f;
                for (int s2 = 16 * j; s2 < 16 * bi; ++s2) x += sA[r * PA + s2] * sT[s2 * PA + col];
                xr[u] = x;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int e = t + u * BT;
            if (u < bi) {
                const int j = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
                sT[(16 * bi + rr) * PA + 16 * j + cc] = xr[u];
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int e = t + u * BT;
            if (u < bi) {
                const int j = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
                float y = 0.f;
                for (int s2 = 0; s2 <= rr; ++s2)
                    y -= sT[(16 * bi + rr) * PA + 16 * bi + s2] * sT[(16 * bi + s2) * PA + 16 * j + cc];
                xr[u] = y;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int e = t + u * BT;
            if (u < bi) {
                const int j = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
                sT[(16 * bi + rr) * PA + 16 * j + cc] = xr[u];
            }
        }
    }
    __syncthreads();   // T complete; Kh' no longer needed
    {
        float* Tg = a.tm + gh * BC * BC;
        for (int e = t; e < BC * BC / 4; e += BT) {
            const int r = e / (BC / 4), c4 = e - r * (BC / 4);
            const float* p = sT + r * PA + 4 * c4;
            *reinterpret_cast<float4*>(Tg + r * BC + 4 * c4) = make_float4(p[0], p[1], p[2], p[3]);
        }
    }
    float* sZ = sKH;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int z = 0; z < 8; ++z) sZ[zr * PZ + sl * BSV + zc + z] = Z[sl][z];
    __syncthreads();
    // Delta = T Z -> global: thread (row zr, 8 columns of each slice)
    {
        float* D = a.dl + gh * BC * DV + (size_t)zr * DV;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
            float acc[8] = {};
            for (int s2 = 0; s2 <= zr; ++s2) {
                const float tt = sT[zr * PA + s2];
#pragma unroll
                for (int z = 0; z < 8; ++z) acc[z] += tt * sZ[s2 * PZ + sl * BSV + zc + z];
            }
#pragma unroll
            for (int z = 0; z < 8; z += 4)
                *reinterpret_cast<float4*>(D + sl * BSV + zc + z) =
                    make_float4(acc[z], acc[z + 1], acc[z + 2], acc[z + 3]);
        }
    }
}

// ---------------------------------------------------------------------------
// per (sequence, head, 32 value columns): the reverse walk carrying dL/dS
// ---------------------------------------------------------------------------
template <typename In, typename Gt, int DK, int DV>
__global__ __launch_bounds__(BT2) void bwd_dstate_kernel(BwdArgs a) {
    constexpr int PE = DK + 1;
    constexpr int PA = BC + 1;
    constexpr int PS = BSV + 1;           // pitch of the [*][32] slabs
    constexpr int CPT = DK * BSV / BT2;   // state columns per thread (8 or 4)
    constexpr int TPR = BSV / CPT;        // threads per state row (4 or 8)
    __shared__ float sKH[BC * PE];
    __shared__ float sQK[BC * PE];        // Qt', then Kt'
    __shared__ float sP[BC * PA];
    __shared__ float sT[BC * PA];
    __shared__ float sDO[BC * PS];        // dO slab
    __shared__ float sDU[DK * PS];        // dU slab
    __shared__ float sDZ[BC * PS];        // dDelta, then dZ slab

    // the slabs of one (sequence, head) on one XCD
    const int units = a.N * a.H;
    const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3;
    const int slab = jj % a.nsl;
    const int pair = (jj / a.nsl) * 8 + xcd;
    if (pair >= units) return;
    const int H = a.H, n = pair / H, h = pair - n * H;
    const int j0 = slab * BSV;
    const int t = threadIdx.x;
    int64_t row0, len;
    seq_of(a, n, row0, len);
    const int64_t nch = (len + BC - 1) / BC;
    const int64_t slot0 = a.coff[n];
    const size_t vst = (size_t)H * DV;
    const In* v = static_cast<const In*>(a.v);
    const In* w = static_cast<const In*>(a.w);
    const In* dout = static_cast<const In*>(a.dout);
    Gt* gdv = static_cast<Gt*>(a.dv);
    Gt* gdw = static_cast<Gt*>(a.dw);

    // running dL/dS: row si, columns j0 + sc .. + CPT - 1
    const int si = t / TPR, sc = (t - si * TPR) * CPT;
    float dN[CPT];
    {
        const size_t sb = ((size_t)pair * DK + si) * DV + j0 + sc;
#pragma unroll
        for (int u = 0; u < CPT; ++u) dN[u] = a.dS_T ? a.dS_T[sb + u] : 0.f;
    }
    // row sum of x over the TPR threads of a state row (adjacent lanes)
    auto row_sum = [&](float x) {
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) x += __shfl_xor(x, o, 64);
        return x;
    };
    // dDelta / dZ layout: row dr, 4 columns dc..
    const int dr = t >> 3, dc = (t & 7) * 4;

    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t g = slot0 + c;
        const size_t gh = (size_t)g * H + h;
        const int clen = (int)min((int64_t)BC, len - c * BC);
        const size_t vb = ((size_t)(row0 + c * BC) * H + h) * DV;
        // ---- S1: stage Kh', Qt', P, T, the dO slab; dU = GR dN; cC ----
        float sn[CPT], scur[CPT];
        {
            const float* Sn = a.ck + ((size_t)(g + 1) * H + h) * DK * DV + (size_t)si * DV + j0 + sc;
            const float* Sc = a.ck + gh * DK * DV + (size_t)si * DV + j0 + sc;
#pragma unroll
            for (int u = 0; u < CPT; u += 4) {
                const float4 x = ld4f(Sn + u), y = ld4f(Sc + u);
                sn[u] = x.x; sn[u + 1] = x.y; sn[u + 2] = x.z; sn[u + 3] = x.w;
                scur[u] = y.x; scur[u + 1] = y.y; scur[u + 2] = y.z; scur[u + 3] = y.w;
            }
        }
        const float gmi = a.gr[gh * 2 * DK + si], gri = a.gr[gh * 2 * DK + DK + si];
        stage<BC, DK, PE, BT2>(sKH, a.kh + gh * BC * DK, DK, BC);
        stage<BC, DK, PE, BT2>(sQK, a.qt + gh * BC * DK, DK, BC);
        stage<BC, BC, PA, BT2>(sP, a.pm + gh * BC * BC, BC, BC);
        stage<BC, BC, PA, BT2>(sT, a.tm + gh * BC * BC, BC, BC);
        stage<BC, BSV, PS, BT2>(sDO, dout + vb + j0, vst, clen);
        float dU[CPT];
        {
            float cc = 0.f;
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                dU[u] = gri * dN[u];
                sDU[si * PS + sc + u] = dU[u];
                cc += dN[u] * sn[u];
            }
            cc = row_sum(cc);
            if (sc == 0) a.cf[((gh * a.nsl + slab) * 2 + 1) * DK + si] = cc;
        }
        __syncthreads();
        // ---- S2: dSm = dU + Qt'^T dO; dDelta = P^T dO + Kh' dU -> sDZ;
        //      Kt' in flight ----
        float ds[CPT];
#pragma unroll
        for (int u = 0; u < CPT; ++u) ds[u] = dU[u];
        for (int r = 0; r < BC; ++r) {
            const float qv = sQK[r * PE + si];
#pragma unroll
            for (int u = 0; u < CPT; ++u) ds[u] += qv * sDO[r * PS + sc + u];
        }
        constexpr int KT4 = BC * DK / 4 / BT2;   // Kt' float4s per thread
        float4 ktr[KT4];
        {
            const float* src = a.kt + gh * BC * DK;
#pragma unroll
            for (int u = 0; u < KT4; ++u) ktr[u] = ld4f(src + 4 * (t + u * BT2));
        }
        {
            float acc[4] = {};
            for (int s2 = dr; s2 < BC; ++s2) {
                const float p = sP[s2 * PA + dr];
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[z] += p * sDO[s2 * PS + dc + z];
            }
            for (int i = 0; i < DK; ++i) {
                const float x = sKH[dr * PE + i];
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[z] += x * sDU[i * PS + dc + z];
            }
#pragma unroll
            for (int z = 0; z < 4; ++z) sDZ[dr * PS + dc + z] = acc[z];
        }
        __syncthreads();
        // ---- S3: dZ = T^T dDelta (registers); Kt' into LDS ----
        float dzr[4] = {};
        for (int s2 = dr; s2 < BC; ++s2) {
            const float tt = sT[s2 * PA + dr];
#pragma unroll
            for (int z = 0; z < 4; ++z) dzr[z] += tt * sDZ[s2 * PS + dc + z];
        }
#pragma unroll
        for (int u = 0; u < KT4; ++u) {
            const int e = t + u * BT2, r = e / (DK / 4), c4 = e - r * (DK / 4);
            st4s(sQK + r * PE + 4 * c4, ktr[u]);
        }
        __syncthreads();
        // ---- S4: dZ -> LDS and the workspace; dv, dw ----
#pragma unroll
        for (int z = 0; z < 4; ++z) sDZ[dr * PS + dc + z] = dzr[z];
        {
            float* Dz = a.dz + gh * BC * DV + (size_t)dr * DV + j0 + dc;
            *reinterpret_cast<float4*>(Dz) = make_float4(dzr[0], dzr[1], dzr[2], dzr[3]);
            if (dr < clen) {
                const size_t o = vb + (size_t)dr * vst + j0 + dc;
                const float4 vv = ld4f(v + o), ww = ld4f(w + o);
                const float xv[4] = {vv.x, vv.y, vv.z, vv.w}, xw[4] = {ww.x, ww.y, ww.z, ww.w};
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    store1(gdw + o + z, dzr[z] * xv[z]);
                    store1(gdv + o + z, dzr[z] * xw[z]);
                }
            }
        }
        __syncthreads();
        // ---- S5: dSm -= Kt'^T dZ; cS = rowsum(dSm Sm); dS = Gm dSm ----
        for (int r = 0; r < BC; ++r) {
            const float kv = sQK[r * PE + si];
#pragma unroll
            for (int u = 0; u < CPT; ++u) ds[u] -= kv * sDZ[r * PS + sc + u];
        }
        {
            float cs = 0.f;
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                cs += ds[u] * (gmi * scur[u]);
                dN[u] = gmi * ds[u];
            }
            cs = row_sum(cs);
            if (sc == 0) a.cf[((gh * a.nsl + slab) * 2 + 0) * DK + si] = cs;
            float* Du = a.du + gh * DK * DV + (size_t)si * DV + j0 + sc;
#pragma unroll
            for (int u = 0; u < CPT; u += 4)
                *reinterpret_cast<float4*>(Du + u) = make_float4(dU[u], dU[u + 1], dU[u + 2], dU[u + 3]);
        }
        __syncthreads();
    }
    if (a.dS0) {
        float* d0 = a.dS0 + ((size_t)pair * DK + si) * DV + j0 + sc;
#pragma unroll
        for (int u = 0; u < CPT; ++u) d0[u] = dN[u];
    }
}

// ---------------------------------------------------------------------------
// per (chunk, head): dq, dk, db, dalpha
// ---------------------------------------------------------------------------
template <typename In, typename Gt, int DK, int DV>
__global__ __launch_bounds__(BT2) void bwd_grad_kernel(BwdArgs a) {
    constexpr int PE = DK + 4;   // float4-aligned rows of the [C][DK] tiles
    constexpr int PA = BC + 1;
    constexpr int PC = BC + 4;   // transposed [32][C] slices
    constexpr int PK = DK + 4;   // transposed [32][DK] slices
    // phase 1 slices, transposed so that a thread's operands are contiguous
    // (dO, dZ, Delta [32][C]; Sm, dU [32][DK]) share the space of phase 2
    // (Kt', Qt', Kh' [C][DK]; dP, dA [C][C])
    constexpr int PH1 = 3 * BSV * PC + 2 * BSV * PK;
    // the tail holds dP and dA, later the [C][DK] coefficients e
    constexpr int PH2 = 3 * BC * PE + (2 * BC * PA > BC * PE ? 2 * BC * PA : BC * PE);
    __shared__ __align__(16) float sm[PH1 > PH2 ? PH1 : PH2];
    __shared__ float sgm[DK], sgr[DK];
    float* sO = sm;
    float* sZ = sO + BSV * PC;
    float* sD = sZ + BSV * PC;
    float* sS = sD + BSV * PC;
    float* sU = sS + BSV * PK;
    float* sKT = sm;
    float* sQT = sKT + BC * PE;
    float* sKH = sQT + BC * PE;
    float* sP = sKH + BC * PE;
    float* sAm = sP + BC * PA;

    const int h = blockIdx.y;
    const int64_t g = blockIdx.x;
    int n;
    int64_t c;
    if (!chunk_of_slot(a, g, n, c)) return;
    const int H = a.H, t = threadIdx.x;
    int64_t row0, len;
    seq_of(a, n, row0, len);
    const int clen = (int)min((int64_t)BC, len - c * BC);
    const size_t kst = (size_t)H * DK, vst = (size_t)H * DV;
    const size_t kb = ((size_t)(row0 + c * BC) * H + h) * DK;
    const size_t vb = ((size_t)(row0 + c * BC) * H + h) * DV;
    const size_t gh = (size_t)g * H + h;
    const In* k = static_cast<const In*>(a.k);
    const In* b = static_cast<const In*>(a.b);
    const In* alpha = static_cast<const In*>(a.alpha);
    const In* dout = static_cast<const In*>(a.dout);

    if (t < DK) sgm[t] = a.gr[gh * 2 * DK + t];
    // thread tiles (8 waves): [C][DK] outputs rows RM*kr.., channels 4 kc..;
    // [C][C] outputs rows 2 pr.., cols 4 pc..
    constexpr int RM = DK / 32;
    constexpr int NKC = DK / 4;
    const int kr = t / NKC, kc = t - kr * NKC;
    const int pr = t >> 4, pc = t & 15;
    float R1[RM][4] = {}, R2[RM][4] = {}, R3[RM][4] = {};
    float dPa[2][4] = {}, dAa[2][4] = {};
    const float* S = a.ck + gh * DK * DV;
    const float* Dg = a.dl + gh * BC * DV;
    const float* Zg = a.dz + gh * BC * DV;
    const float* Ug = a.du + gh * DK * DV;
    __syncthreads();
    // ---- phase 1: products over the value axis, 32 columns at a time ----
    for (int j0 = 0; j0 < DV; j0 += BSV) {
        stage_t<BC, BSV, PC, BT2>(sO, dout + vb + j0, vst, clen);
        stage_t<BC, BSV, PC, BT2>(sZ, Zg + j0, DV, BC);
        stage_t<BC, BSV, PC, BT2>(sD, Dg + j0, DV, BC);
        stage_t<DK, BSV, PK, BT2>(sS, S + j0, DV, DK, sgm);
        stage_t<DK, BSV, PK, BT2>(sU, Ug + j0, DV, DK);
        __syncthreads();
        for (int jj = 0; jj < BSV; ++jj) {
            float so[RM], sz[RM], sd[RM];
#pragma unroll
            for (int u = 0; u < RM; ++u) {
                so[u] = sO[jj * PC + RM * kr + u];
                sz[u] = sZ[jj * PC + RM * kr + u];
                sd[u] = sD[jj * PC + RM * kr + u];
            }
            const float4 s4 = *reinterpret_cast<const float4*>(sS + jj * PK + 4 * kc);
            const float4 u4 = *reinterpret_cast<const float4*>(sU + jj * PK + 4 * kc);
            const float ss[4] = {s4.x, s4.y, s4.z, s4.w}, su[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
            for (int u = 0; u < RM; ++u)
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    R1[u][z] += so[u] * ss[z];
                    R2[u][z] += sz[u] * ss[z];
                    R3[u][z] += sd[u] * su[z];
                }
            const float po[2] = {sO[jj * PC + 2 * pr], sO[jj * PC + 2 * pr + 1]};
            const float pz[2] = {sZ[jj * PC + 2 * pr], sZ[jj * PC + 2 * pr + 1]};
            const float4 d4 = *reinterpret_cast<const float4*>(sD + jj * PC + 4 * pc);
            const float pd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    dPa[u][z] += po[u] * pd[z];
                    dAa[u][z] += pz[u] * pd[z];
                }
        }
        __syncthreads();
    }
    // ---- phase 2: tiles, dP = tril(dO Delta^T), dA = -strictly_lower(dZ Delta^T) ----
    stage<BC, DK, PE, BT2>(sKT, a.kt + gh * BC * DK, DK, BC);
    stage<BC, DK, PE, BT2>(sQT, a.qt + gh * BC * DK, DK, BC);
    stage<BC, DK, PE, BT2>(sKH, a.kh + gh * BC * DK, DK, BC);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            const int r = 2 * pr + u, s2 = 4 * pc + z;
            sP[r * PA + s2] = s2 <= r ? dPa[u][z] : 0.f;
            sAm[r * PA + s2] = s2 < r ? -dAa[u][z] : 0.f;
        }
    __syncthreads();
    // dQt' = R1 + dP Kh';  dKt' = -R2 + dA Kh';  dKh' = R3 + dP^T Qt' + dA^T Kt'
#pragma unroll
    for (int u = 0; u < RM; ++u)
#pragma unroll
        for (int z = 0; z < 4; ++z) R2[u][z] = -R2[u][z];
    for (int s2 = 0; s2 < BC; ++s2) {
        const float4 h4 = *reinterpret_cast<const float4*>(sKH + s2 * PE + 4 * kc);
        const float4 q4 = *reinterpret_cast<const float4*>(sQT + s2 * PE + 4 * kc);
        const float4 t4 = *reinterpret_cast<const float4*>(sKT + s2 * PE + 4 * kc);
        const float kh[4] = {h4.x, h4.y, h4.z, h4.w}, qt[4] = {q4.x, q4.y, q4.z, q4.w},
                    kt[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
        for (int u = 0; u < RM; ++u) {
            const int r = RM * kr + u;
            const float p_rs = sP[r * PA + s2], a_rs = sAm[r * PA + s2];
            const float p_sr = sP[s2 * PA + r], a_sr = sAm[s2 * PA + r];
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                R1[u][z] += p_rs * kh[z];
                R2[u][z] += a_rs * kh[z];
                R3[u][z] += p_sr * qt[z] + a_sr * kt[z];
            }
        }
    }
    // e = dKt' Kt' + dQt' Qt' - dKh' Kh'
    float ev[RM][4];
#pragma unroll
    for (int u = 0; u < RM; ++u)
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            const int r = RM * kr + u, i = 4 * kc + z;
            ev[u][z] = R2[u][z] * sKT[r * PE + i] + R1[u][z] * sQT[r * PE + i] -
                       R3[u][z] * sKH[r * PE + i];
        }
    __syncthreads();
    // e into the dP / dA space ([C][DK], pitch PE); the factors e1
    float* sEv = sP;
#pragma unroll
    for (int u = 0; u < RM; ++u)
#pragma unroll
        for (int z = 0; z < 4; ++z) sEv[(RM * kr + u) * PE + 4 * kc + z] = ev[u][z];
    chunk_factors<In, DK, PE>(alpha, kb, kst, clen, sKT, sgm, sgr);
    __syncthreads();
    // dq = dQt' e1; db = dKt' k e1; dk = dKt' b e1 + dKh' / e1
    {
        Gt* gq = static_cast<Gt*>(a.dq);
        Gt* gk = static_cast<Gt*>(a.dk);
        Gt* gb = static_cast<Gt*>(a.db);
#pragma unroll
        for (int u = 0; u < RM; ++u) {
            const int r = RM * kr + u;
            if (r >= clen) continue;
            const size_t o = kb + (size_t)r * kst + 4 * kc;
            const float4 k4 = ld4f(k + o), b4 = ld4f(b + o);
            const float xk[4] = {k4.x, k4.y, k4.z, k4.w}, xb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const float e1 = sKT[r * PE + 4 * kc + z];
                store1(gq + o + z, R1[u][z] * e1);
                store1(gb + o + z, R2[u][z] * xk[z] * e1);
                store1(gk + o + z, R2[u][z] * xb[z] * e1 + R3[u][z] / e1);
            }
        }
    }
    // dalpha: suffix sums of e over the rows, one thread per key channel
    if (t < DK) {
        const int i = t;
        float tot = 0.f;
        for (int r = 0; r < BC; ++r) tot += sEv[r * PE + i];
        float cS = 0.f, cC = 0.f;
        for (int sl = 0; sl < a.nsl; ++sl) {
            cS += a.cf[((gh * a.nsl + sl) * 2 + 0) * DK + i];
            cC += a.cf[((gh * a.nsl + sl) * 2 + 1) * DK + i];
        }
        const float cm = cS - cC - tot;
        Gt* ga = static_cast<Gt*>(a.dalpha);
        float suf = 0.f;
        for (int r = BC - 1; r >= 0; --r) {
            suf += sEv[r * PE + i];
            if (r < clen) {
                const size_t o = kb + (size_t)r * kst + i;
                const float dl = suf + (r <= BMID ? cm : 0.f) + cC;
                store1(ga + o, dl / ldf(alpha + o));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

struct BwdLayout {
    size_t fwd_ws, coff, ck, kt, qt, kh, pm, tm, dl, gr, du, dz, cf, total;
    int64_t slots;
    int nsl;
};

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

BwdLayout bwd_layout(int B, int T, int H, int dk, int dv, int num_seqs, int in_dtype) {
    BwdLayout L;
    const bool packed = B == 1 && num_seqs > 1;
    const int64_t N = packed ? num_seqs : B;
    const int64_t nch = ((int64_t)T + BC - 1) / BC;
    L.slots = packed ? (int64_t)T / BC + 2 * N + 1 : N * (nch + 1);
    L.nsl = dv / BSV;
    const FwdPlan fp = plan_fwd(B, T, H, dk, dv, num_seqs, in_dtype);
    const size_t u = (size_t)L.slots * H;
    size_t o = 0;
    L.fwd_ws = o; o += al256(fp.workspace);
    L.coff = o;   o += al256((size_t)(N + 1) * sizeof(int64_t));
    L.ck = o;     o += al256(u * dk * dv * 4);
    L.kt = o;     o += al256(u * BC * dk * 4);
    L.qt = o;     o += al256(u * BC * dk * 4);
    L.kh = o;     o += al256(u * BC * dk * 4);
    L.pm = o;     o += al256(u * BC * BC * 4);
    L.tm = o;     o += al256(u * BC * BC * 4);
    L.dl = o;     o += al256(u * BC * dv * 4);
    L.gr = o;     o += al256(u * 2 * dk * 4);
    L.du = o;     o += al256(u * dk * dv * 4);
    L.dz = o;     o += al256(u * BC * dv * 4);
    L.cf = o;     o += al256(u * L.nsl * 2 * dk * 4);
    L.total = o;
    return L;
}

template <typename In, typename Gt, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs& a, int64_t slots, hipStream_t stream) {
    const dim3 gchunks((unsigned)slots, (unsigned)a.H);
    hipLaunchKernelGGL((bwd_prep_kernel<In, DK, DV>), gchunks, dim3(BT), 0, stream, a);
    // slabs of one (sequence, head) on one XCD: groups of 8 units
    const unsigned groups = (unsigned)((a.N * a.H + 7) / 8);
    hipLaunchKernelGGL((bwd_dstate_kernel<In, Gt, DK, DV>), dim3(groups * 8 * a.nsl), dim3(BT2),
                       0, stream, a);
    hipLaunchKernelGGL((bwd_grad_kernel<In, Gt, DK, DV>), gchunks, dim3(BT2), 0, stream, a);
    return hipGetLastError();
}

template <typename In, typename Gt>
hipError_t launch_bwd_d(const BwdArgs& a, int64_t slots, int dk, int dv, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_bwd_t<In, Gt, 128, 128>(a, slots, stream);
    if (dk == 128 && dv == 64) return launch_bwd_t<In, Gt, 128, 64>(a, slots, stream);
    if (dk == 64 && dv == 128) return launch_bwd_t<In, Gt, 64, 128>(a, slots, stream);
    return launch_bwd_t<In, Gt, 64, 64>(a, slots, stream);
}

}  // namespace

size_t bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs, int in_dtype) {
    return bwd_layout(B, T, H, dk, dv, num_seqs, in_dtype).total;
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* alpha,
                      const void* b, const void* w, int in_dtype, const float* S0,
                      const void* dout, const float* dS_T, void* dq, void* dk, void* dv,
                      void* dalpha, void* db, void* dw, int grad_dtype, float* dS0,
                      const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int dkd,
                      int dvd, void* workspace, hipStream_t stream) {
    const BwdLayout L = bwd_layout(B, T, H, dkd, dvd, num_seqs, in_dtype);
    const int N = cu_seqlens ? num_seqs : B;
    if (N == 0) return hipSuccess;
    char* ws = static_cast<char*>(workspace);
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.b = b; a.w = w; a.dout = dout;
    a.S0 = S0; a.dS_T = dS_T;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dalpha = dalpha; a.db = db; a.dw = dw; a.dS0 = dS0;
    a.cu = cu_seqlens; a.N = N; a.T = T; a.H = H;
    a.coff = reinterpret_cast<int64_t*>(ws + L.coff);
    float* ck = reinterpret_cast<float*>(ws + L.ck);
    a.ck = ck;
    a.kt = reinterpret_cast<float*>(ws + L.kt);
    a.qt = reinterpret_cast<float*>(ws + L.qt);
    a.kh = reinterpret_cast<float*>(ws + L.kh);
    a.pm = reinterpret_cast<float*>(ws + L.pm);
    a.tm = reinterpret_cast<float*>(ws + L.tm);
    a.dl = reinterpret_cast<float*>(ws + L.dl);
    a.gr = reinterpret_cast<float*>(ws + L.gr);
    a.du = reinterpret_cast<float*>(ws + L.du);
    a.dz = reinterpret_cast<float*>(ws + L.dz);
    a.cf = reinterpret_cast<float*>(ws + L.cf);
    a.nsl = L.nsl;
    hipLaunchKernelGGL(bwd_slots_kernel, dim3(1), dim3(BT), 0, stream, cu_seqlens, N, T,
                       reinterpret_cast<int64_t*>(ws + L.coff));
    // the forward in checkpoint mode: chunk start states and final states
    const FwdPlan fp = plan_fwd(B, T, H, dkd, dvd, num_seqs, in_dtype);
    hipError_t e = launch_fwd(fp, q, k, v, alpha, b, w, in_dtype, S0, nullptr, DT_F32, nullptr,
                              cu_seqlens, num_seqs, B, T, H, dkd, dvd, GATES_FULL,
                              ws + L.fwd_ws, stream, ck);
    if (e != hipSuccess) return e;
    if (in_dtype == DT_BF16) {
        if (grad_dtype == DT_BF16) return launch_bwd_d<bf16_t, bf16_t>(a, L.slots, dkd, dvd, stream);
        return launch_bwd_d<bf16_t, float>(a, L.slots, dkd, dvd, stream);
    }
    return launch_bwd_d<float, float>(a, L.slots, dkd, dvd, stream);
}

}  // namespace gdn2
