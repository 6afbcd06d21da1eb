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
//   bwd_prep_kernel   per (chunk, head): A, P, T = (I + A)^-1 (column
//                     substitution), Delta, and the per-channel Gm, GR
//   bwd_dstate_kernel per (sequence, head, 32 value columns): the reverse
//                     walk over chunks carrying dL/dS; stores dU and dZ per
//                     chunk, writes dv, dw and dS0, and the row sums cS, cC
//   bwd_grad_kernel   per (chunk, head): the products over the value axis and
//                     the chunk axis above, then dq, dk, db, dalpha
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

constexpr int BC = 64;        // chunk length
constexpr int BMID = 31;      // midpoint row of a chunk
constexpr int BT = 256;       // threads per workgroup
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
    if (per == 0 && t == 0) coff[N] = 0;
}

// ---------------------------------------------------------------------------
// per (chunk, head): A, P, T = (I + A)^-1, Delta, Gm, GR
// ---------------------------------------------------------------------------
template <typename In, int DK, int DV>
__global__ __launch_bounds__(BT) void bwd_prep_kernel(BwdArgs a) {
    constexpr int PE = DK + 1;   // pitch of the [C][DK] tiles
    constexpr int PA = BC + 1;   // pitch of the [C][C] tiles
    constexpr int PZ = DV + 1;   // pitch of Z
    __shared__ float sE[BC * PE];    // e1, then Kt', then Qt'
    __shared__ float sKH[BC * (PE > PZ ? PE : PZ)];   // Kh', then Z = X - Kt' Sm
    __shared__ float sA[BC * PA];
    __shared__ float sT[BC * PA];
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
    // Kh' = k / e1 and Kt' = b k e1 (over e1, element by element)
    for (int e = t; e < BC * DK; e += BT) {
        const int r = e / DK, i = e - r * DK;
        const bool ok = r < clen;
        const float kk = ok ? ldf(k + kb + (size_t)r * kst + i) : 0.f;
        const float bb = ok ? ldf(b + kb + (size_t)r * kst + i) : 0.f;
        const float e1 = sE[r * PE + i];
        sKH[r * PE + i] = kk / e1;
        sE[r * PE + i] = bb * kk * e1;
    }
    __syncthreads();
    // A = strictly_lower(Kt' Kh'^T): thread (rows 4 tr.., cols 4 tc..)
    {
        const int tr = t >> 4, tc = t & 15;
        float acc[4][4] = {};
        for (int i = 0; i < DK; ++i) {
            float x[4], y[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[u] = sE[(4 * tr + u) * PE + i];
                y[u] = sKH[(4 * tc + u) * PE + i];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[u][z] += x[u] * y[z];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int r = 4 * tr + u, s = 4 * tc + z;
                sA[r * PA + s] = s < r ? acc[u][z] : 0.f;
            }
    }
    // Y = Kt' Sm (Sm = Gm (.) S from the checkpoint); Z = X - Y in registers:
    // thread (rows TM zr.., cols 4 zc..)
    constexpr int TM = DV / 16;          // rows per thread
    constexpr int NCB = DV / 4;          // column blocks
    const int zr = t / NCB, zc = t - zr * NCB;
    float Z[TM][4] = {};
    {
        const float* S = a.ck + gh * DK * DV;
        for (int i = 0; i < DK; ++i) {
            const float gmi = sgm[i];
            const float4 s4 = *reinterpret_cast<const float4*>(S + (size_t)i * DV + 4 * zc);
            const float sv[4] = {s4.x * gmi, s4.y * gmi, s4.z * gmi, s4.w * gmi};
#pragma unroll
            for (int u = 0; u < TM; ++u) {
                const float x = sE[(TM * zr + u) * PE + i];
#pragma unroll
                for (int z = 0; z < 4; ++z) Z[u][z] -= x * sv[z];
            }
        }
#pragma unroll
        for (int u = 0; u < TM; ++u) {
            const int r = TM * zr + u;
            if (r < clen) {
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    const size_t o = vb + (size_t)r * vst + 4 * zc + z;
                    Z[u][z] += ldf(w + o) * ldf(v + o);
                }
            }
        }
    }
    __syncthreads();
    // Qt' = q e1 over Kt' (e1 = Kt' / (b k) is gone: recompute from the factors)
    chunk_factors<In, DK, PE>(static_cast<const In*>(a.alpha), kb, kst, clen, sE, sgm, sgr);
    __syncthreads();
    for (int e = t; e < BC * DK; e += BT) {
        const int r = e / DK, i = e - r * DK;
        const float qq = r < clen ? ldf(q + kb + (size_t)r * kst + i) : 0.f;
        sE[r * PE + i] *= qq;
    }
    __syncthreads();
    // P = tril(Qt' Kh'^T) -> global
    {
        const int tr = t >> 4, tc = t & 15;
        float acc[4][4] = {};
        for (int i = 0; i < DK; ++i) {
            float x[4], y[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[u] = sE[(4 * tr + u) * PE + i];
                y[u] = sKH[(4 * tc + u) * PE + i];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[u][z] += x[u] * y[z];
        }
        float* P = a.pm + gh * BC * BC;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int r = 4 * tr + u, s = 4 * tc + z;
                P[r * BC + s] = s <= r ? acc[u][z] : 0.f;
            }
    }
    // T = (I + A)^-1 by forward substitution, one column per thread
    if (t < BC) {
        const int j = t;
        for (int r = 0; r < BC; ++r) {
            float x = 0.f;
            if (r == j) x = 1.f;
            else if (r > j) {
                for (int s = j; s < r; ++s) x -= sA[r * PA + s] * sT[s * PA + j];
            }
            sT[r * PA + j] = x;
        }
    }
    __syncthreads();   // T complete; Kh' no longer needed
    {
        float* Tg = a.tm + gh * BC * BC;
        for (int e = t; e < BC * BC; e += BT) Tg[e] = sT[(e / BC) * PA + (e % BC)];
    }
    float* sZ = sKH;
#pragma unroll
    for (int u = 0; u < TM; ++u)
#pragma unroll
        for (int z = 0; z < 4; ++z) sZ[(TM * zr + u) * PZ + 4 * zc + z] = Z[u][z];
    __syncthreads();
    // Delta = T Z -> global
    {
        float acc[TM][4] = {};
        for (int s = 0; s < BC; ++s) {
            float zz[4];
#pragma unroll
            for (int z = 0; z < 4; ++z) zz[z] = sZ[s * PZ + 4 * zc + z];
#pragma unroll
            for (int u = 0; u < TM; ++u) {
                const float tt = sT[(TM * zr + u) * PA + s];
#pragma unroll
                for (int z = 0; z < 4; ++z) acc[u][z] += tt * zz[z];
            }
        }
        float* D = a.dl + gh * BC * DV;
#pragma unroll
        for (int u = 0; u < TM; ++u)
            *reinterpret_cast<float4*>(D + (size_t)(TM * zr + u) * DV + 4 * zc) =
                make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
    }
}

// ---------------------------------------------------------------------------
// per (sequence, head, 32 value columns): the reverse walk carrying dL/dS
// ---------------------------------------------------------------------------
template <typename In, typename Gt, int DK, int DV>
__global__ __launch_bounds__(BT) void bwd_dstate_kernel(BwdArgs a) {
    constexpr int PE = DK + 1;
    constexpr int PS = BSV + 1;           // pitch of the [*][32] slabs
    constexpr int CPT = DK * BSV / BT;    // state columns per thread (16 or 8)
    constexpr int TPR = BSV / CPT;        // threads per state row (2 or 4)
    __shared__ float sKT[BC * PE];        // e1, then Kt'
    __shared__ float sKH[BC * PE];
    __shared__ float sQT[BC * PE];
    __shared__ float sDO[BC * PS];        // dO slab
    __shared__ float sDU[DK * PS];        // dU slab
    __shared__ float sDZ[BC * PS];        // dDelta, then dZ slab
    __shared__ float sgm[DK], sgr[DK];

    const int pair = blockIdx.x / a.nsl;
    const int slab = blockIdx.x - pair * a.nsl;
    const int H = a.H, n = pair / H, h = pair - n * H;
    const int j0 = slab * BSV;
    const int t = threadIdx.x;
    int64_t row0, len;
    seq_of(a, n, row0, len);
    const int64_t nch = (len + BC - 1) / BC;
    const int64_t slot0 = a.coff[n];
    const size_t kst = (size_t)H * DK, vst = (size_t)H * DV;
    const In* q = static_cast<const In*>(a.q);
    const In* k = static_cast<const In*>(a.k);
    const In* v = static_cast<const In*>(a.v);
    const In* b = static_cast<const In*>(a.b);
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

    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t g = slot0 + c;
        const size_t gh = (size_t)g * H + h;
        const int clen = (int)min((int64_t)BC, len - c * BC);
        const size_t kb = ((size_t)(row0 + c * BC) * H + h) * DK;
        const size_t vb = ((size_t)(row0 + c * BC) * H + h) * DV;
        chunk_factors<In, DK, PE>(static_cast<const In*>(a.alpha), kb, kst, clen, sKT, sgm, sgr);
        // dO slab
        for (int e = t; e < BC * BSV; e += BT) {
            const int r = e / BSV, jj = e - r * BSV;
            sDO[r * PS + jj] = r < clen ? ldf(dout + vb + (size_t)r * vst + j0 + jj) : 0.f;
        }
        __syncthreads();
        // tiles over e1: Kh' = k / e1, Qt' = q e1, Kt' = b k e1
        for (int e = t; e < BC * DK; e += BT) {
            const int r = e / DK, i = e - r * DK;
            const bool ok = r < clen;
            const size_t o = kb + (size_t)r * kst + i;
            const float kk = ok ? ldf(k + o) : 0.f;
            const float qq = ok ? ldf(q + o) : 0.f;
            const float bb = ok ? ldf(b + o) : 0.f;
            const float e1 = sKT[r * PE + i];
            sKH[r * PE + i] = kk / e1;
            sQT[r * PE + i] = qq * e1;
            sKT[r * PE + i] = bb * kk * e1;
        }
        // dU = GR dN into LDS; cC = rowsum(dN S_next) (S_next = next checkpoint)
        {
            const float gri = sgr[si];
            const float* Sn = a.ck + ((size_t)(g + 1) * H + h) * DK * DV + (size_t)si * DV + j0 + sc;
            float cc = 0.f;
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                sDU[si * PS + sc + u] = gri * dN[u];
                cc += dN[u] * Sn[u];
            }
            cc = row_sum(cc);
            if (sc == 0) a.cf[((gh * a.nsl + slab) * 2 + 1) * DK + si] = cc;
        }
        __syncthreads();
        // dDelta = P^T dO + Kh' dU: thread (row dr, 8 columns dc..)
        const int dr = t >> 2, dc = (t & 3) * 8;
        {
            const float* P = a.pm + gh * BC * BC;
            float acc[8] = {};
            for (int s = dr; s < BC; ++s) {
                const float p = P[s * BC + dr];
#pragma unroll
                for (int z = 0; z < 8; ++z) acc[z] += p * sDO[s * PS + dc + z];
            }
            for (int i = 0; i < DK; ++i) {
                const float x = sKH[dr * PE + i];
#pragma unroll
                for (int z = 0; z < 8; ++z) acc[z] += x * sDU[i * PS + dc + z];
            }
#pragma unroll
            for (int z = 0; z < 8; ++z) sDZ[dr * PS + dc + z] = acc[z];
        }
        __syncthreads();
        // dZ = T^T dDelta
        float dzr[8] = {};
        {
            const float* Tm = a.tm + gh * BC * BC;
            for (int s = dr; s < BC; ++s) {
                const float tt = Tm[s * BC + dr];
#pragma unroll
                for (int z = 0; z < 8; ++z) dzr[z] += tt * sDZ[s * PS + dc + z];
            }
        }
        __syncthreads();
#pragma unroll
        for (int z = 0; z < 8; ++z) sDZ[dr * PS + dc + z] = dzr[z];
        {
            float* Dz = a.dz + gh * BC * DV + (size_t)dr * DV + j0 + dc;
#pragma unroll
            for (int z = 0; z < 8; z += 4)
                *reinterpret_cast<float4*>(Dz + z) = make_float4(dzr[z], dzr[z + 1], dzr[z + 2], dzr[z + 3]);
            if (dr < clen) {
                const size_t o = vb + (size_t)dr * vst + j0 + dc;
#pragma unroll
                for (int z = 0; z < 8; ++z) {
                    store1(gdw + o + z, dzr[z] * ldf(v + o + z));
                    store1(gdv + o + z, dzr[z] * ldf(w + o + z));
                }
            }
        }
        __syncthreads();
        // dSm = Qt'^T dO + dU - Kt'^T dZ; cS = rowsum(dSm Sm); dS = Gm dSm
        {
            float ds[CPT];
#pragma unroll
            for (int u = 0; u < CPT; ++u) ds[u] = sDU[si * PS + sc + u];
            for (int r = 0; r < BC; ++r) {
                const float qv = sQT[r * PE + si], kv = sKT[r * PE + si];
#pragma unroll
                for (int u = 0; u < CPT; ++u)
                    ds[u] += qv * sDO[r * PS + sc + u] - kv * sDZ[r * PS + sc + u];
            }
            const float gmi = sgm[si];
            const float* Sc = a.ck + gh * DK * DV + (size_t)si * DV + j0 + sc;
            float cs = 0.f;
#pragma unroll
            for (int u = 0; u < CPT; ++u) {
                cs += ds[u] * (gmi * Sc[u]);
                dN[u] = gmi * ds[u];
            }
            cs = row_sum(cs);
            if (sc == 0) a.cf[((gh * a.nsl + slab) * 2 + 0) * DK + si] = cs;
            // dU slab -> global
            float* Du = a.du + gh * DK * DV + (size_t)si * DV + j0 + sc;
#pragma unroll
            for (int u = 0; u < CPT; ++u) Du[u] = sDU[si * PS + sc + u];
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
__global__ __launch_bounds__(BT) void bwd_grad_kernel(BwdArgs a) {
    constexpr int PE = DK + 1;
    constexpr int PA = BC + 1;
    constexpr int PS = BSV + 1;
    // phase 1 slices (dO, dZ, Delta [C][32]; Sm, dU [DK][32]) share the
    // space of phase 2 (Kt', Qt', Kh' [C][DK]; dP, dA [C][C])
    constexpr int PH1 = 3 * BC * PS + 2 * DK * PS;
    constexpr int PH2 = 3 * BC * PE + 2 * BC * PA;
    __shared__ float sm[PH1 > PH2 ? PH1 : PH2];
    __shared__ float sgm[DK], sgr[DK];
    float* sO = sm;
    float* sZ = sO + BC * PS;
    float* sD = sZ + BC * PS;
    float* sS = sD + BC * PS;
    float* sU = sS + DK * PS;
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
    const In* q = static_cast<const In*>(a.q);
    const In* k = static_cast<const In*>(a.k);
    const In* b = static_cast<const In*>(a.b);
    const In* alpha = static_cast<const In*>(a.alpha);
    const In* dout = static_cast<const In*>(a.dout);

    if (t < DK) sgm[t] = a.gr[gh * 2 * DK + t];
    // thread tiles: [C][DK] outputs rows RM*kr.., channels 4 kc..; [C][C]
    // outputs rows 4 pr.., cols 4 pc..
    constexpr int RM = DK / 16;
    constexpr int NKC = DK / 4;
    const int kr = t / NKC, kc = t - kr * NKC;
    const int pr = t >> 4, pc = t & 15;
    float R1[RM][4] = {}, R2[RM][4] = {}, R3[RM][4] = {};
    float dPa[4][4] = {}, dAa[4][4] = {};
    const float* S = a.ck + gh * DK * DV;
    const float* Dg = a.dl + gh * BC * DV;
    const float* Zg = a.dz + gh * BC * DV;
    const float* Ug = a.du + gh * DK * DV;
    __syncthreads();
    // ---- phase 1: products over the value axis, 32 columns at a time ----
    for (int j0 = 0; j0 < DV; j0 += BSV) {
        for (int e = t; e < BC * BSV; e += BT) {
            const int r = e / BSV, jj = e - r * BSV;
            sO[r * PS + jj] = r < clen ? ldf(dout + vb + (size_t)r * vst + j0 + jj) : 0.f;
            sZ[r * PS + jj] = Zg[(size_t)r * DV + j0 + jj];
            sD[r * PS + jj] = Dg[(size_t)r * DV + j0 + jj];
        }
        for (int e = t; e < DK * BSV; e += BT) {
            const int i = e / BSV, jj = e - i * BSV;
            sS[i * PS + jj] = sgm[i] * S[(size_t)i * DV + j0 + jj];
            sU[i * PS + jj] = Ug[(size_t)i * DV + j0 + jj];
        }
        __syncthreads();
        for (int jj = 0; jj < BSV; ++jj) {
            float so[RM], sz[RM], sd[RM], ss[4], su[4];
#pragma unroll
            for (int u = 0; u < RM; ++u) {
                so[u] = sO[(RM * kr + u) * PS + jj];
                sz[u] = sZ[(RM * kr + u) * PS + jj];
                sd[u] = sD[(RM * kr + u) * PS + jj];
            }
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                ss[z] = sS[(4 * kc + z) * PS + jj];
                su[z] = sU[(4 * kc + z) * PS + jj];
            }
#pragma unroll
            for (int u = 0; u < RM; ++u)
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    R1[u][z] += so[u] * ss[z];
                    R2[u][z] += sz[u] * ss[z];
                    R3[u][z] += sd[u] * su[z];
                }
            float po[4], pz[4], pd[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                po[u] = sO[(4 * pr + u) * PS + jj];
                pz[u] = sZ[(4 * pr + u) * PS + jj];
                pd[u] = sD[(4 * pc + u) * PS + jj];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    dPa[u][z] += po[u] * pd[z];
                    dAa[u][z] += pz[u] * pd[z];
                }
        }
        __syncthreads();
    }
    // ---- phase 2: tiles, dP = tril(dO Delta^T), dA = -strictly_lower(dZ Delta^T) ----
    chunk_factors<In, DK, PE>(alpha, kb, kst, clen, sKT, sgm, sgr);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            const int r = 4 * pr + u, s = 4 * pc + z;
            sP[r * PA + s] = s <= r ? dPa[u][z] : 0.f;
            sAm[r * PA + s] = s < r ? -dAa[u][z] : 0.f;
        }
    __syncthreads();
    for (int e = t; e < BC * DK; e += BT) {
        const int r = e / DK, i = e - r * DK;
        const bool ok = r < clen;
        const size_t o = kb + (size_t)r * kst + i;
        const float kk = ok ? ldf(k + o) : 0.f;
        const float qq = ok ? ldf(q + o) : 0.f;
        const float bb = ok ? ldf(b + o) : 0.f;
        const float e1 = sKT[r * PE + i];
        sKH[r * PE + i] = kk / e1;
        sQT[r * PE + i] = qq * e1;
        sKT[r * PE + i] = bb * kk * e1;
    }
    __syncthreads();
    // dQt' = R1 + dP Kh';  dKt' = -R2 + dA Kh';  dKh' = R3 + dP^T Qt' + dA^T Kt'
    for (int u = 0; u < RM; ++u)
#pragma unroll
        for (int z = 0; z < 4; ++z) R2[u][z] = -R2[u][z];
    for (int s = 0; s < BC; ++s) {
        float kh[4], qt[4], kt[4];
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            kh[z] = sKH[s * PE + 4 * kc + z];
            qt[z] = sQT[s * PE + 4 * kc + z];
            kt[z] = sKT[s * PE + 4 * kc + z];
        }
#pragma unroll
        for (int u = 0; u < RM; ++u) {
            const int r = RM * kr + u;
            const float p_rs = sP[r * PA + s], a_rs = sAm[r * PA + s];
            const float p_sr = sP[s * PA + r], a_sr = sAm[s * PA + r];
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
    // e into the dP space ([C][DK], pitch PE: fits dP + dA); factors again
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
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int i = 4 * kc + z;
                const size_t o = kb + (size_t)r * kst + i;
                const float e1 = sKT[r * PE + i];
                const float kk = ldf(k + o), bb = ldf(b + o);
                store1(gq + o, R1[u][z] * e1);
                store1(gb + o, R2[u][z] * kk * e1);
                store1(gk + o, R2[u][z] * bb * e1 + R3[u][z] / e1);
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
    size_t fwd_ws, coff, ck, pm, tm, dl, gr, du, dz, cf, total;
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
    hipLaunchKernelGGL((bwd_dstate_kernel<In, Gt, DK, DV>), dim3((unsigned)(a.N * a.H * a.nsl)),
                       dim3(BT), 0, stream, a);
    hipLaunchKernelGGL((bwd_grad_kernel<In, Gt, DK, DV>), gchunks, dim3(BT), 0, stream, a);
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
