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
// Kernels (all arithmetic fp32, the products on fp32 MFMA; the forward runs
// first in its checkpoint mode, storing every chunk's start state):
//   bwd_slots_kernel  slot offsets of the sequences' chunks (packed batches)
//   bwd_prep_kernel   per (chunk, head), 16 waves: the tiles Kt', Qt', Kh',
//                     A, P, T = (I + A)^-1 (16x16 diagonal blocks by the
//                     doubling product, the rest by block columns), Delta,
//                     and Gm, GR
//   bwd_dstate_kernel per (sequence, head, 64 value columns), 16 waves: the
//                     reverse walk over chunks carrying dL/dS; stores dU and
//                     dZ per chunk, writes dv, dw and dS0, and the row sums
//                     cS, cC.  The column slabs of one (sequence, head) run
//                     on one XCD, so they share the chunk's tiles in its L2.
//   bwd_grad_kernel   per (chunk, head), 16 waves: the products over the
//                     value axis and the chunk axis above, then dq, dk, db,
//                     dalpha
// Global loads are issued well before their data is needed (whole blocks
// held in registers, stored to LDS at the next phase); the products read
// LDS only.
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

namespace gdn2 {

namespace {

constexpr int BC = 64;        // chunk length
constexpr int BMID = 31;      // midpoint row of a chunk
constexpr int BT = 256;       // threads per workgroup (prep, grad)
constexpr int BT3 = 1024;     // threads per workgroup (prep, gradients)
constexpr int DT = 512;       // threads per workgroup (reverse walk)
constexpr int BSV = 32;       // value columns per slice of the gradient kernel's phase 1
constexpr int DSV = 64;       // value columns per reverse-walk workgroup

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
    float* cf;             // [slot][H][dv/16][2][dk]  cS, cC partial row sums per 16-column tile
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

// fp32 MFMA on 16 x 16 tiles, 16 contraction indices per call: lane (m =
// l & 15, g = l >> 4) supplies A[m][k0 + 4g + e] and B^T[n = m][k0 + 4g + e]
// for e = 0 .. 3 (the same permutation of the contraction index on both
// sides), loaded by frag4 as one float4 from a row-major LDS tile whose
// pitch is 4 (mod 32) floats, which keeps the reads conflict-free.  The
// output holds D[4g + j][l & 15] in element j.
__device__ __forceinline__ float4 frag4(const float* base, int pitch, int row0, int k0, int l) {
    return *reinterpret_cast<const float4*>(base + (row0 + (l & 15)) * pitch + k0 + 4 * (l >> 4));
}
__device__ __forceinline__ floatx4 mma4x(float4 a, float4 b, floatx4 c) {
    c = mma16(a.x, b.x, c);
    c = mma16(a.y, b.y, c);
    c = mma16(a.z, b.z, c);
    return mma16(a.w, b.w, c);
}
// X Y for 16 x 16 register tiles, X given as the accumulator tile of X^T
// (whose layout is the A-operand layout of X) and Y as its accumulator tile
// (the B-operand layout, contraction index 4g + j in step j).
__device__ __forceinline__ floatx4 prod32(floatx4 XtAcc, floatx4 YAcc, floatx4 C) {
#pragma unroll
    for (int j = 0; j < 4; ++j) C = mma16(XtAcc[j], YAcc[j], C);
    return C;
}
// (I + N)^-1 of a 16 x 16 block, N strictly lower (N^16 = 0), from the
// accumulator tiles of N and N^T: (I - N)(I + N^2)(I + N^4)(I + N^8).
__device__ __forceinline__ floatx4 diag_inverse32(floatx4 N, floatx4 Nt, int l) {
    const int g4 = l >> 4, ln = l & 15;
    const floatx4 z = zero4();
    const floatx4 N2 = prod32(Nt, N, z);
    const floatx4 N2t = prod32(N, Nt, z);
    const floatx4 N4 = prod32(N2t, N2, z);
    const floatx4 N4t = prod32(N2, N2t, z);
    const floatx4 N8t = prod32(N4, N4t, z);
    floatx4 Z;
#pragma unroll
    for (int j = 0; j < 4; ++j) Z[j] = ((4 * g4 + j == ln) ? 1.f : 0.f) - N[j];
    Z = prod32(N2t, Z, Z);
    Z = prod32(N4t, Z, Z);
    Z = prod32(N8t, Z, Z);
    return Z;
}
// acc + A B for 16 x 16 blocks: A rows a_row .., columns a_col .. of a
// row-major LDS array; B an accumulator tile.
__device__ __forceinline__ floatx4 blk32(floatx4 acc, const float* A, int apitch, int a_row,
                                         int a_col, floatx4 B, int l) {
    const float* pa = A + (a_row + (l & 15)) * apitch + a_col + 4 * (l >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mma16(pa[j], B[j], acc);
    return acc;
}
// The same fragment from a row-major tile whose rows are the contraction
// index: lane (n = l & 15, g) gathers B[k0 + 4g + e][n0 + n], e = 0 .. 3.
__device__ __forceinline__ float4 frag_col(const float* base, int pitch, int k0, int n0, int l) {
    const float* p = base + (k0 + 4 * (l >> 4)) * pitch + n0 + (l & 15);
    return make_float4(p[0], p[pitch], p[2 * pitch], p[3 * pitch]);
}

// A ROWS x COLS block of a row-major global array, held in registers by the
// NTH threads of a workgroup (float4 e = t + u NTH: row e / (COLS / 4)),
// so that its loads can be issued well before it is stored to LDS.  Rows at
// or past `valid` read as zero.
template <int ROWS, int COLS, int NTH>
struct Rows {
    static constexpr int C4 = COLS / 4, N4 = ROWS * C4, PER = (N4 + NTH - 1) / NTH;
    float4 x[PER];
    template <typename Src>
    __device__ __forceinline__ void load(const Src* src, size_t stride, int valid) {
        const int t = threadIdx.x;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = t + u * NTH;
            const int r = e / C4, c = e - r * C4;
            x[u] = (e < N4 && r < valid) ? ld4f(src + (size_t)r * stride + 4 * c) : zf4();
        }
    }
    // to LDS with row pitch `pitch` (a multiple of 4), times rowscale[r]
    // when given
    __device__ __forceinline__ void store(float* dst, int pitch, const float* rowscale = nullptr) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = t + u * NTH;
            if (e < N4) {
                const int r = e / C4, c = e - r * C4;
                float4 v = x[u];
                if (rowscale) {
                    const float sc = rowscale[r];
                    v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
                }
                *reinterpret_cast<float4*>(dst + r * pitch + 4 * c) = v;
            }
        }
    }
};

// Storage words of 4 consecutive elements, widened to fp32 only where they
// are used.  A bf16 load whose widening sits right after it (inside the
// branch of a row check, or in the same block) needs a wait on the spot, and
// on this hardware that wait (vmcnt) counts the workgroup's earlier stores
// too: every such load waited for all of them to land.
template <typename In>
struct Raw4;
template <>
struct Raw4<float> {
    float4 v;
};
template <>
struct Raw4<bf16_t> {
    uint2 v;
};
__device__ __forceinline__ void ld_raw4(const float* p, Raw4<float>& r) {
    r.v = *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ void ld_raw4(const bf16_t* p, Raw4<bf16_t>& r) {
    r.v = *reinterpret_cast<const uint2*>(p);
}
__device__ __forceinline__ float4 widen4(const Raw4<float>& r) { return r.v; }
__device__ __forceinline__ float4 widen4(const Raw4<bf16_t>& r) {
    return make_float4(__uint_as_float(r.v.x << 16), __uint_as_float(r.v.x & 0xffff0000u),
                       __uint_as_float(r.v.y << 16), __uint_as_float(r.v.y & 0xffff0000u));
}
// one element: the loaded bits (bf16 in the low half) or the fp32 value
__device__ __forceinline__ uint32_t ld_raw1(const bf16_t* p) { return p->bits; }
__device__ __forceinline__ float ld_raw1(const float* p) { return *p; }
__device__ __forceinline__ float widen1(uint32_t bits) { return __uint_as_float(bits << 16); }
__device__ __forceinline__ float widen1(float x) { return x; }
template <typename In>
using RawEl = decltype(ld_raw1(static_cast<const In*>(nullptr)));

// Rows for a block of the input dtype with a runtime row count: rows at or
// past `valid` (>= 1) are loaded from row 0 (in range, no branch) and stored
// to LDS as zero; the words stay raw until the store.
template <int ROWS, int COLS, int NTH, typename In>
struct RowsIn {
    static constexpr int C4 = COLS / 4, N4 = ROWS * C4, PER = (N4 + NTH - 1) / NTH;
    Raw4<In> x[PER];
    int valid;
    __device__ __forceinline__ void load(const In* src, size_t stride, int valid_) {
        valid = valid_;
        const int t = threadIdx.x;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = t + u * NTH;
            const int r = e / C4, c = e - r * C4;
            if (e < N4) ld_raw4(src + (size_t)(r < valid_ ? r : 0) * stride + 4 * c, x[u]);
        }
    }
    __device__ __forceinline__ void store(float* dst, int pitch) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = t + u * NTH;
            if (e < N4) {
                const int r = e / C4, c = e - r * C4;
                const float4 v = r < valid ? widen4(x[u]) : zf4();
                *reinterpret_cast<float4*>(dst + r * pitch + 4 * c) = v;
            }
        }
    }
};

// Decay factors of one run of RPT rows r0 .. r0 + RPT - 1 of a chunk for
// one key channel (the run lies on one side of the midpoint row 31): e1_r =
// 1 / prod_{s in (r, 31]} alpha_s below the midpoint, prod_{s in (31, r]}
// alpha_s above it, with the products taken outwards from the midpoint.
// `own` holds the run's alphas, `ext` those of the rows between the run and
// the midpoint (ext[u] = row r0 + RPT + u below, row 32 + u above; 1 past
// the rows it spans).  Also returns the product over the whole half when the
// run reaches the chunk's edge: gamma_mid (run starting at row 0) or
// gamma_C / gamma_mid (run ending at row 63).
template <int RPT>
struct RunFactors {
    float own[RPT], ext[32 - RPT], e1[RPT], half;
    template <typename In>
    __device__ __forceinline__ void load(const In* alpha, size_t base, size_t rstride, int r0, int clen) {
        const bool lo = r0 <= BMID;
        const int e0 = lo ? r0 + RPT : BMID + 1;       // first ext row
        const int ne = lo ? BMID + 1 - e0 : r0 - e0;   // ext rows
        // every load first, from row 0 where the row is absent (no branch),
        // then the widening: a conditional load widened in its own branch
        // waited for that load before the next one was issued
        RawEl<In> ro[RPT], rx[32 - RPT];
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int r = r0 + u;
            ro[u] = ld_raw1(alpha + base + (size_t)(r < clen ? r : 0) * rstride);
        }
#pragma unroll
        for (int u = 0; u < 32 - RPT; ++u) {
            const int r = e0 + u;
            rx[u] = ld_raw1(alpha + base + (size_t)((u < ne && r < clen) ? r : 0) * rstride);
        }
#pragma unroll
        for (int u = 0; u < RPT; ++u) own[u] = r0 + u < clen ? widen1(ro[u]) : 1.f;
#pragma unroll
        for (int u = 0; u < 32 - RPT; ++u) ext[u] = (u < ne && e0 + u < clen) ? widen1(rx[u]) : 1.f;
    }
    __device__ __forceinline__ void factors(int r0) {
        if (r0 <= BMID) {
            float p = 1.f;
#pragma unroll
            for (int u = 31 - RPT; u >= 0; --u) p *= ext[u];
#pragma unroll
            for (int u = RPT - 1; u >= 0; --u) {
                e1[u] = 1.f / p;
                p *= own[u];
            }
            half = p;
        } else {
            float qv = 1.f;
#pragma unroll
            for (int u = 0; u < 32 - RPT; ++u) qv *= ext[u];
#pragma unroll
            for (int u = 0; u < RPT; ++u) {
                qv *= own[u];
                e1[u] = qv;
            }
            half = qv;
        }
    }
};

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
// 8 waves; every global load is issued at the start.
//   1. thread (channel i, run of RPT rows): decay factors e1 of its rows from
//      the alphas between them and the midpoint, the tiles Kt', Qt', Kh' of
//      its rows (LDS and the workspace); Gm and GR.
//   2. fp32 MFMA: waves 0-3 the diagonal blocks A_ww, A_ww^T, P_ww; waves 4-7
//      the off-diagonal A blocks (4, 5) and P blocks (6, 7), three each.  A
//      goes to LDS, P to the workspace.  Waves 0-3 invert their diagonal
//      block in registers: (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8).
//   3. Sm = Gm (.) S into LDS; wave J forms block column J of T from the
//      diagonal blocks: T_iJ = -T_ii sum_{m=J}^{i-1} A_im T_mJ.
//   4. Z = X - Kt' Sm (rows rt, half of the value columns per wave), into
//      LDS over Sm; Delta = T Z to the workspace; T to the workspace.
template <typename In, int DK, int DV>
__global__ __launch_bounds__(BT3) void bwd_prep_kernel(BwdArgs a) {
    constexpr int PE = DK + 4;   // [C][DK] tiles
    constexpr int PC = BC + 4;   // [C][C] tiles
    constexpr int PV = DV + 4;   // [DK][DV] Sm, then [C][DV] Z
    constexpr int RPT = BC * DK / BT3;
    constexpr int RG = BT3 / DK;
    static_assert(RPT % 4 == 0 && 32 % RPT == 0, "row runs");
    constexpr int NJ = DV / 64;  // value-column tiles per wave
    constexpr int OFF_KT = 0, OFF_QT = BC * PE, OFF_KH = 2 * BC * PE;
    constexpr int OFF_S = BC * PE;                 // Sm over Qt', Kh' (free after step 2)
    constexpr int OFF_A = 3 * BC * PE > OFF_S + DK * PV ? 3 * BC * PE : OFF_S + DK * PV;
    constexpr int OFF_T = OFF_A + BC * PC;
    constexpr int SM = OFF_T + BC * PC;
    static_assert(BC * PV <= DK * PV, "Z over Sm");
    __shared__ __align__(16) float sm[SM];
    __shared__ float sgm[DK];

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
    const In* v = static_cast<const In*>(a.v);
    const In* w = static_cast<const In*>(a.w);
    const int wv = t >> 6, l = t & 63, g4 = l >> 4, ln = l & 15;
    // step 4: row tile rt and value-column quarter jh; the four waves on one
    // SIMD (wv mod 4) take the four row tiles
    const int rt = (wv + (wv >> 2)) & 3;
    const int jh = wv >> 2;

    // ---- loads ----
    const int i = t % DK, rg = t / DK, r0 = RPT * rg;
    // loads unconditional (absent rows read row 0) and widened after all
    // of them are out
    RawEl<In> rq[RPT], rk[RPT], rbk[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int r = r0 + u;
        const size_t o = kb + (size_t)(r < clen ? r : 0) * kst + i;
        rq[u] = ld_raw1(q + o);
        rk[u] = ld_raw1(k + o);
        rbk[u] = ld_raw1(b + o);
    }
    RunFactors<RPT> rf;
    rf.load(alpha, kb + i, kst, r0, clen);
    float xq[RPT], xk[RPT], xb[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const bool ok = r0 + u < clen;
        xq[u] = ok ? widen1(rq[u]) : 0.f;
        xk[u] = ok ? widen1(rk[u]) : 0.f;
        xb[u] = ok ? widen1(rbk[u]) : 0.f;
    }
    Rows<DK, DV, BT3> rS;
    rS.load(a.ck + gh * DK * DV, DV, DK);
    // X = w (.) v at the positions of the Z tiles (rows 16 rt + 4 g + jj,
    // columns 32 jh + 16 ... + ln)
    RawEl<In> rw[NJ][4], rv[NJ][4];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = 16 * rt + 4 * g4 + jj, col = 16 * (NJ * jh + jt) + ln;
            const size_t o = vb + (size_t)(r < clen ? r : 0) * vst + col;
            rw[jt][jj] = ld_raw1(w + o);
            rv[jt][jj] = ld_raw1(v + o);
        }
    float xv[NJ][4];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            xv[jt][jj] = 16 * rt + 4 * g4 + jj < clen ? widen1(rw[jt][jj]) * widen1(rv[jt][jj]) : 0.f;
    for (int e = t; e < BC * PC; e += BT3) sm[OFF_T + e] = 0.f;

    // ---- step 1: decay factors and tiles ----
    {
        rf.factors(r0);
        const float* e1 = rf.e1;
        if (rg == 0) {
            sgm[i] = rf.half;
            a.gr[gh * 2 * DK + i] = rf.half;
        }
        if (rg == RG - 1) a.gr[gh * 2 * DK + DK + i] = rf.half;
        float* gkt = a.kt + gh * BC * DK;
        float* gqt = a.qt + gh * BC * DK;
        float* gkh = a.kh + gh * BC * DK;
#pragma unroll
        for (int u = 0; u < RPT; ++u) {
            const int r = r0 + u;
            const float kt = xb[u] * xk[u] * e1[u], qt = xq[u] * e1[u], kh = xk[u] / e1[u];
            sm[OFF_KT + r * PE + i] = kt;
            sm[OFF_QT + r * PE + i] = qt;
            sm[OFF_KH + r * PE + i] = kh;
            gkt[r * DK + i] = kt;
            gqt[r * DK + i] = qt;
            gkh[r * DK + i] = kh;
        }
    }
    __syncthreads();
    // ---- step 2: A, P; diagonal inverses ----
    floatx4 Tdiag = zero4();
    {
        float* gP = a.pm + gh * BC * BC;
        auto store_p = [&](int R, int S2, floatx4 x, bool mask) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * R + 4 * g4 + jj, s2 = 16 * S2 + ln;
                gP[r * BC + s2] = (!mask || s2 <= r) ? x[jj] : 0.f;
            }
        };
        if (wv < 4) {
            // A_ww (N), A_ww^T (Nt) and P_ww share their fragments
            floatx4 N = zero4(), Nt = zero4(), Pd = zero4();
#pragma unroll 4
            for (int kk = 0; kk < DK / 16; ++kk) {
                const float4 fkt = frag4(sm + OFF_KT, PE, 16 * wv, 16 * kk, l);
                const float4 fkh = frag4(sm + OFF_KH, PE, 16 * wv, 16 * kk, l);
                const float4 fq = frag4(sm + OFF_QT, PE, 16 * wv, 16 * kk, l);
                N = mma4x(fkt, fkh, N);
                Nt = mma4x(fkh, fkt, Nt);
                Pd = mma4x(fq, fkh, Pd);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rr = 4 * g4 + jj;
                N[jj] = rr > ln ? N[jj] : 0.f;
                Nt[jj] = ln > rr ? Nt[jj] : 0.f;
                sm[OFF_A + (16 * wv + rr) * PC + 16 * wv + ln] = N[jj];
            }
            store_p(wv, wv, Pd, true);
            for (int S2 = wv + 1; S2 < 4; ++S2) store_p(wv, S2, zero4(), false);
            Tdiag = diag_inverse32(N, Nt, l);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                sm[OFF_T + (16 * wv + 4 * g4 + jj) * PC + 16 * wv + ln] = Tdiag[jj];
        } else if (wv < 8) {
            // waves 4, 5: A_10 A_20 A_30 | A_21 A_31 A_32; waves 6, 7: the same P
            const bool isP = wv >= 6;
            const int S2 = (wv & 1);
            const int R0 = S2 + 1;
            floatx4 acc[3] = {zero4(), zero4(), zero4()};
            const int nr = 3 - S2;
#pragma unroll 4
            for (int kk = 0; kk < DK / 16; ++kk) {
                const float4 fb = frag4(sm + OFF_KH, PE, 16 * S2, 16 * kk, l);
#pragma unroll
                for (int x = 0; x < 3; ++x) {
                    if (x < nr) {
                        const float4 fa = frag4(sm + (isP ? OFF_QT : OFF_KT), PE, 16 * (R0 + x), 16 * kk, l);
                        acc[x] = mma4x(fa, fb, acc[x]);
                    }
                }
            }
            if (wv == 5 || wv == 7) {
                // second column set: (2,1), (3,1), (3,2): the last block has S = 2
                floatx4 acc2 = zero4();
#pragma unroll 4
                for (int kk = 0; kk < DK / 16; ++kk) {
                    const float4 fb = frag4(sm + OFF_KH, PE, 32, 16 * kk, l);
                    const float4 fa = frag4(sm + (isP ? OFF_QT : OFF_KT), PE, 48, 16 * kk, l);
                    acc2 = mma4x(fa, fb, acc2);
                }
                acc[2] = acc2;
            }
            // blocks: wave 4/6 (R, 0) for R = 1..3; wave 5/7 (2,1), (3,1), (3,2)
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                const int R = (wv & 1) ? (x < 2 ? 2 + x : 3) : 1 + x;
                const int Sx = (wv & 1) ? (x < 2 ? 1 : 2) : 0;
                if (isP) {
                    store_p(R, Sx, acc[x], false);
                } else {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        sm[OFF_A + (16 * R + 4 * g4 + jj) * PC + 16 * Sx + ln] = acc[x][jj];
                }
            }
        }
    }
    __syncthreads();   // A and the diagonal blocks of T in LDS; Qt', Kh' free
    // ---- step 3: Sm; block columns of T ----
    rS.store(sm + OFF_S, PV, sgm);
    if (wv < 3) {
        // column J = wv: T_iJ for i = J + 1 .. 3, from T_JJ (registers)
        const int J = wv;
        floatx4 Tc[4];
        Tc[0] = Tc[1] = Tc[2] = Tc[3] = zero4();
        Tc[J] = Tdiag;
        for (int i2 = J + 1; i2 < 4; ++i2) {
            floatx4 X = zero4();
            for (int m = J; m < i2; ++m) X = blk32(X, sm + OFF_A, PC, 16 * i2, 16 * m, Tc[m], l);
            const floatx4 Y = blk32(zero4(), sm + OFF_T, PC, 16 * i2, 16 * i2, X, l);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                Tc[i2][jj] = -Y[jj];
                sm[OFF_T + (16 * i2 + 4 * g4 + jj) * PC + 16 * J + ln] = -Y[jj];
            }
        }
    }
    __syncthreads();
    // ---- step 4: Z = X - Kt' Sm; Delta = T Z ----
    floatx4 Z[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) Z[jt] = zero4();
#pragma unroll 4
    for (int kk = 0; kk < DK / 16; ++kk) {
        const float4 fa = frag4(sm + OFF_KT, PE, 16 * rt, 16 * kk, l);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            const float4 fb = frag_col(sm + OFF_S, PV, 16 * kk, 16 * (NJ * jh + jt), l);
            Z[jt] = mma4x(fa, fb, Z[jt]);
        }
    }
    {
        // T to the workspace (complete since the last barrier)
        float* gT = a.tm + gh * BC * BC;
        for (int e = t; e < BC * BC / 4; e += BT3) {
            const int r = e / (BC / 4), c4 = e - r * (BC / 4);
            *reinterpret_cast<float4*>(gT + r * BC + 4 * c4) =
                *reinterpret_cast<const float4*>(sm + OFF_T + r * PC + 4 * c4);
        }
    }
    __syncthreads();   // every wave is done with Sm
    float* sZ = sm + OFF_S;
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            sZ[(16 * rt + 4 * g4 + jj) * PV + 16 * (NJ * jh + jt) + ln] = xv[jt][jj] - Z[jt][jj];
    __syncthreads();
    floatx4 D[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) D[jt] = zero4();
    for (int sb = 0; sb <= rt; ++sb) {
        const float4 fa = frag4(sm + OFF_T, PC, 16 * rt, 16 * sb, l);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            const float4 fb = frag_col(sZ, PV, 16 * sb, 16 * (NJ * jh + jt), l);
            D[jt] = mma4x(fa, fb, D[jt]);
        }
    }
    float* gD = a.dl + gh * BC * DV;
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            gD[(16 * rt + 4 * g4 + jj) * DV + 16 * (NJ * jh + jt) + ln] = D[jt][jj];
}

// ---------------------------------------------------------------------------
// per (sequence, head, 64 value columns): the reverse walk carrying dL/dS
// ---------------------------------------------------------------------------
// DT / 64 waves, fp32 MFMA.  The running dN = dL/dS (DK x 64) lives in
// registers: wave w holds tiles x = TPW w .. (row tile x / 4, column tile
// x % 4).  Per chunk, from the last to the first:
//   A: dU = GR dN (LDS and workspace), cC; dDelta = P^T dO + Kh' dU, wave w
//      the tiles (row tile rt, column tiles jt0 ..)
//   B: dZ = T^T dDelta, the same tile split; dZ to LDS and the workspace,
//      dv = dZ w, dw = dZ v
//   C: dSm = Qt'^T dO + dU - Kt'^T dZ on the state tiles; cS; dN = Gm dSm
// The next chunk's operands are loaded into registers during A (P, T, Kh',
// dO, GR), during B (Qt', Kt') and after C (S_c, Gm, v, w: the registers
// are free by then).  cS and cC go out as partial row sums per 16-column
// tile.  (16 waves measured slower: the 128-register limit spills.)
template <typename In, typename Gt, int DK, int DV>
__global__ __launch_bounds__(DT) void bwd_dstate_kernel(BwdArgs a) {
    constexpr int PJ = DSV + 4;
    constexpr int PC = BC + 4;
    constexpr int PE = DK + 4;
    constexpr int NI = DK / 16;
    constexpr int NJD = DSV / 16;       // column tiles of the slab
    constexpr int NW = DT / 64;         // waves
    constexpr int TPW = NI * NJD / NW;  // state tiles per wave
    constexpr int NTW = 4 * NJD / NW;   // dDelta / dZ tiles per wave
    static_assert(TPW >= 1, "state tiles");
    // LDS regions
    constexpr int OFF_O = 0;                           // dO [C][PJ]
    constexpr int OFF_R1 = OFF_O + BC * PJ;            // Kh' (A), then Qt' (C)
    constexpr int OFF_R2 = OFF_R1 + BC * PE;           // P [C][PC] + dU [DK][PJ] (A), then Kt' (C)
    constexpr int R2N = BC * PC + DK * PJ > BC * PE ? BC * PC + DK * PJ : BC * PE;
    constexpr int OFF_R3 = OFF_R2 + R2N;               // T [C][PC] + dDelta [C][PJ]
    constexpr int OFF_DZ = OFF_R3 + BC * PC + BC * PJ; // dZ [C][PJ]
    constexpr int SM = OFF_DZ + BC * PJ;
    __shared__ __align__(16) float sm[SM];
    float* const sO = sm + OFF_O;
    float* const sKh = sm + OFF_R1;
    float* const sQ = sm + OFF_R1;
    float* const sP = sm + OFF_R2;
    float* const sDU = sm + OFF_R2 + BC * PC;
    float* const sKt = sm + OFF_R2;
    float* const sT = sm + OFF_R3;
    float* const sDD = sm + OFF_R3 + BC * PC;
    float* const sDZ = sm + OFF_DZ;

    // the slabs of one (sequence, head) on one XCD
    const int units = a.N * a.H;
    const int xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
    const int slab = jb % a.nsl;
    const int pair = (jb / a.nsl) * 8 + xcd;
    if (pair >= units) return;
    const int H = a.H, n = pair / H, h = pair - n * H;
    const int j0 = slab * DSV;
    const int t = threadIdx.x;
    const int wv = t >> 6, l = t & 63, g4 = l >> 4, ln = l & 15;
    // the dDelta / dZ tiles of the wave: row tile rt, column tiles jt0 ..
    // jt0 + NTW - 1; the waves on one SIMD (wv mod 4) take complementary row
    // tiles, which evens out the triangular products
    const int rt = NW == 16 ? (wv + (wv >> 2)) & 3 : (wv < 4 ? wv : 7 - wv);
    const int jt0 = NTW * (wv >> 2);
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
    const int ncf = DV / 16;   // partial row sums per (slot, head): one per 16-column tile

    // state tile u of the wave: rows 16 I + 4 g + jj, columns j0 + 16 J + ln
    auto tI = [&](int u) { return (TPW * wv + u) / NJD; };
    auto tJ = [&](int u) { return (TPW * wv + u) % NJD; };
    floatx4 dN[TPW];
    #pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            dN[u][jj] = a.dS_T ? a.dS_T[((size_t)pair * DK + 16 * tI(u) + 4 * g4 + jj) * DV + j0 +
                                        16 * tJ(u) + ln]
                               : 0.f;
    if (nch == 0) {
        if (a.dS0)
    #pragma unroll
            for (int u = 0; u < TPW; ++u)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    a.dS0[((size_t)pair * DK + 16 * tI(u) + 4 * g4 + jj) * DV + j0 + 16 * tJ(u) + ln] = dN[u][jj];
        return;
    }

    // ---- operands in registers ----
    Rows<BC, BC, DT> rP, rT;
    Rows<BC, DK, DT> rKh, rQ, rKt;
    RowsIn<BC, DSV, DT, In> rO;
    // the wave's state tiles share their rows: 16 rI + 4 g + jj
    static_assert(TPW <= NJD, "state tiles of a wave in one row tile");
    const int rI = tI(0);
    float scur[TPW][4], snext[TPW][4], gmv[4], grv[4];
    RawEl<In> xv[NTW][4], xw[NTW][4];   // raw v, w at the dZ tile (widened at the use)
    auto state_vals = [&](int64_t g, float (&dst)[TPW][4]) {
        const float* S = a.ck + ((size_t)g * H + h) * DK * DV;
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                dst[u][jj] = S[(size_t)(16 * rI + 4 * g4 + jj) * DV + j0 + 16 * tJ(u) + ln];
    };
    // loaded one chunk ahead, used in stage A: P, T, Kh', dO, GR
    auto load_a = [&](int64_t c) {
        const int64_t g = slot0 + c;
        const size_t gh = (size_t)g * H + h;
        const int clen = (int)min((int64_t)BC, len - c * BC);
        rP.load(a.pm + gh * BC * BC, BC, BC);
        rT.load(a.tm + gh * BC * BC, BC, BC);
        rKh.load(a.kh + gh * BC * DK, DK, BC);
        const size_t vb = ((size_t)(row0 + c * BC) * H + h) * DV;
        rO.load(dout + vb + j0, vst, clen);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) grv[jj] = a.gr[gh * 2 * DK + DK + 16 * rI + 4 * g4 + jj];
    };
    // loaded in stage B, used in stage C: Qt', Kt'
    auto load_c = [&](int64_t c) {
        const size_t gh = (size_t)(slot0 + c) * H + h;
        rQ.load(a.qt + gh * BC * DK, DK, BC);
        rKt.load(a.kt + gh * BC * DK, DK, BC);
    };
    // loaded at the end of the previous chunk (after its last use of the
    // same registers): S_c, Gm, and v, w at the dZ tile
    auto load_late = [&](int64_t c) {
        const int64_t g = slot0 + c;
        const size_t gh = (size_t)g * H + h;
        const int clen = (int)min((int64_t)BC, len - c * BC);
        state_vals(g, scur);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) gmv[jj] = a.gr[gh * 2 * DK + 16 * rI + 4 * g4 + jj];
        const size_t vb = ((size_t)(row0 + c * BC) * H + h) * DV;
#pragma unroll
        for (int x = 0; x < NTW; ++x)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                // rows past the chunk's end read row 0 (their products are
                // not stored)
                const int r = 16 * rt + 4 * g4 + jj;
                const size_t o = vb + (size_t)(r < clen ? r : 0) * vst + j0 + 16 * (jt0 + x) + ln;
                xv[x][jj] = ld_raw1(v + o);
                xw[x][jj] = ld_raw1(w + o);
            }
    };
    state_vals(slot0 + nch, snext);   // the final state
    load_a(nch - 1);
    load_c(nch - 1);
    load_late(nch - 1);

    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t g = slot0 + c;
        const size_t gh = (size_t)g * H + h;
        const int clen = (int)min((int64_t)BC, len - c * BC);
        const size_t vb = ((size_t)(row0 + c * BC) * H + h) * DV;
        // ---- stage A; dU = GR dN; cC ----
        rP.store(sP, PC);
        rT.store(sT, PC);
        rKh.store(sKh, PE);
        rO.store(sO, PJ);
        floatx4 dU[TPW];
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                dU[u][jj] = grv[jj] * dN[u][jj];
                const int i = 16 * tI(u) + 4 * g4 + jj, j = 16 * tJ(u) + ln;
                sDU[i * PJ + j] = dU[u][jj];
                a.du[gh * DK * DV + (size_t)i * DV + j0 + j] = dU[u][jj];
                float cc = dN[u][jj] * snext[u][jj];
                cc += __shfl_xor(cc, 1, 64);
                cc += __shfl_xor(cc, 2, 64);
                cc += __shfl_xor(cc, 4, 64);
                cc += __shfl_xor(cc, 8, 64);
                if (ln == 0) a.cf[((gh * ncf + NJD * slab + tJ(u)) * 2 + 1) * DK + i] = cc;
            }
        __syncthreads();
        if (c > 0) load_a(c - 1);
        // ---- A: dDelta tiles (rt, jt0 + x) = P^T dO + Kh' dU ----
        {
            floatx4 acc[NTW];
#pragma unroll
            for (int x = 0; x < NTW; ++x) acc[x] = zero4();
            for (int rb = rt; rb < BC / 16; ++rb) {
                const float4 fp = frag_col(sP, PC, 16 * rb, 16 * rt, l);
#pragma unroll
                for (int x = 0; x < NTW; ++x)
                    acc[x] = mma4x(fp, frag_col(sO, PJ, 16 * rb, 16 * (jt0 + x), l), acc[x]);
            }
#pragma unroll
            for (int kb2 = 0; kb2 < NI; ++kb2) {
                const float4 fk = frag4(sKh, PE, 16 * rt, 16 * kb2, l);
#pragma unroll
                for (int x = 0; x < NTW; ++x)
                    acc[x] = mma4x(fk, frag_col(sDU, PJ, 16 * kb2, 16 * (jt0 + x), l), acc[x]);
            }
#pragma unroll
            for (int x = 0; x < NTW; ++x)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    sDD[(16 * rt + 4 * g4 + jj) * PJ + 16 * (jt0 + x) + ln] = acc[x][jj];
        }
        __syncthreads();
        // ---- stage C's tiles; B: dZ tiles (rt, jt0 + x) = T^T dDelta ----
        rQ.store(sQ, PE);
        rKt.store(sKt, PE);
        if (c > 0) load_c(c - 1);
        {
            floatx4 acc[NTW];
#pragma unroll
            for (int x = 0; x < NTW; ++x) acc[x] = zero4();
            for (int sb = rt; sb < BC / 16; ++sb) {
                const float4 ft = frag_col(sT, PC, 16 * sb, 16 * rt, l);
#pragma unroll
                for (int x = 0; x < NTW; ++x)
                    acc[x] = mma4x(ft, frag_col(sDD, PJ, 16 * sb, 16 * (jt0 + x), l), acc[x]);
            }
#pragma unroll
            for (int x = 0; x < NTW; ++x)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = 16 * rt + 4 * g4 + jj, j = 16 * (jt0 + x) + ln;
                    sDZ[r * PJ + j] = acc[x][jj];
                    a.dz[gh * BC * DV + (size_t)r * DV + j0 + j] = acc[x][jj];
                    if (r < clen) {
                        const size_t o = vb + (size_t)r * vst + j0 + j;
                        store1(gdw + o, acc[x][jj] * widen1(xv[x][jj]));
                        store1(gdv + o, acc[x][jj] * widen1(xw[x][jj]));
                    }
                }
        }
        __syncthreads();
        // ---- C: dSm = Qt'^T dO + dU - Kt'^T dZ; cS; dN = Gm dSm ----
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            floatx4 pq = zero4(), pk = zero4();
#pragma unroll
            for (int rb = 0; rb < BC / 16; ++rb) {
                const float4 fo = frag_col(sO, PJ, 16 * rb, 16 * tJ(u), l);
                const float4 fz = frag_col(sDZ, PJ, 16 * rb, 16 * tJ(u), l);
                pq = mma4x(frag_col(sQ, PE, 16 * rb, 16 * tI(u), l), fo, pq);
                pk = mma4x(frag_col(sKt, PE, 16 * rb, 16 * tI(u), l), fz, pk);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float ds = pq[jj] + dU[u][jj] - pk[jj];
                float cs = ds * (gmv[jj] * scur[u][jj]);
                cs += __shfl_xor(cs, 1, 64);
                cs += __shfl_xor(cs, 2, 64);
                cs += __shfl_xor(cs, 4, 64);
                cs += __shfl_xor(cs, 8, 64);
                const int i = 16 * tI(u) + 4 * g4 + jj;
                if (ln == 0) a.cf[((gh * ncf + NJD * slab + tJ(u)) * 2 + 0) * DK + i] = cs;
                dN[u][jj] = gmv[jj] * ds;
            }
        }
        // S_c is the next chunk's S_next; then the late loads of that chunk
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) snext[u][jj] = scur[u][jj];
        if (c > 0) load_late(c - 1);
        __syncthreads();
    }
    if (a.dS0)
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                a.dS0[((size_t)pair * DK + 16 * tI(u) + 4 * g4 + jj) * DV + j0 + 16 * tJ(u) + ln] = dN[u][jj];
}

// ---------------------------------------------------------------------------
// per (chunk, head): dq, dk, db, dalpha
// ---------------------------------------------------------------------------
// Every product runs on fp32 MFMA (16 x 16 tiles, contraction 4 per
// instruction; see mma4x).  Wave w owns row tile rt of the chunk (rows
// 16 rt ..) and channel half ch (channel tiles NCH ch ..); waves w and w + 4
// share a SIMD and take row tiles rt and 3 - rt, which evens out the
// triangular products.
//   phase 1, over the value axis in 32-column slices (the next slice's loads
//   in flight while the current one is multiplied):
//     R1 = dO Sm^T, R2 = dZ Sm^T (rows rt, the wave's channels),
//     R3 = Delta dU^T (rows rt as the s index, the wave's channels),
//     dP = dO Delta^T, dA = dZ Delta^T on the lower tiles (rt, S), S <= rt,
//     S = ch (mod 2)
//   phase 2 (Kh', Qt', Kt' loaded during the last slice):
//     dQt' = R1 + dP Kh', dKt' = -R2 + dA Kh'    (contraction s <= r)
//     dKh' = R3 + dP^T Qt' + dA^T Kt'            (contraction r >= s)
//   epilogue, one thread per (channel, run of RPT rows): its decay factors
//     from the alphas, dq, dk, db and e; dalpha by suffix sums of e over the
//     rows, the later runs' sums shared through LDS.
template <typename In, typename Gt, int DK, int DV>
__global__ __launch_bounds__(BT3) void bwd_grad_kernel(BwdArgs a) {
    constexpr int PJ = BSV + 4;   // pitch of the phase-1 slices ([*][32])
    constexpr int PC = BC + 4;    // pitch of the [*][C] tiles
    constexpr int PE = DK + 4;    // pitch of the [C][DK] tiles
    constexpr int NCH = DK / 64;  // channel tiles per wave
    // phase 1: dO, dZ, Delta slices [C][PJ]; Sm, dU slices [DK][PJ]
    constexpr int OFF_O = 0, OFF_Z = BC * PJ, OFF_D = 2 * BC * PJ, OFF_S = 3 * BC * PJ;
    constexpr int OFF_U = OFF_S + DK * PJ;
    constexpr int P1 = OFF_U + DK * PJ;
    // phase 2: dP, dA [C][PC]; Kh', Qt', Kt' [C][PE]
    constexpr int OFF_P = 0, OFF_A = BC * PC, OFF_KH = 2 * BC * PC;
    constexpr int OFF_QT = OFF_KH + BC * PE, OFF_KT = OFF_QT + BC * PE;
    constexpr int P2 = OFF_KT + BC * PE;
    // epilogue: dQt'^T, dKt'^T, dKh'^T [DK][PC]; per-run sums of e [RG][DK]
    constexpr int RPT = BC * DK / BT3;   // rows per epilogue thread
    constexpr int RG = BT3 / DK;         // runs of rows
    static_assert(RPT % 4 == 0 && 32 % RPT == 0, "epilogue runs");
    constexpr int OFF_SUM = 3 * DK * PC;
    constexpr int P3 = OFF_SUM + RG * DK;
    constexpr int SM = P1 > P2 ? (P1 > P3 ? P1 : P3) : (P2 > P3 ? P2 : P3);
    __shared__ __align__(16) float sm[SM];
    __shared__ float sgm[DK];

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

    // 16 waves: wave w takes row tile rt and channel quarter ch; the four
    // waves on one SIMD (w mod 4) take all four row tiles
    const int w = t >> 6, l = t & 63, g4 = l >> 4, ln = l & 15;
    const int rt = (w + (w >> 2)) & 3;
    const int ch = w >> 2;
    auto ctile = [&](int ct) { return 16 * (NCH * ch + ct); };   // first channel of a tile

    if (t < DK) sgm[t] = a.gr[gh * 2 * DK + t];
    // the lower tile (rt, ch) of dP and dA, when ch <= rt
    floatx4 R1[NCH], R2[NCH], R3[NCH], dPa, dAa;
#pragma unroll
    for (int ct = 0; ct < NCH; ++ct) R1[ct] = R2[ct] = R3[ct] = zero4();
    dPa = dAa = zero4();
    const float* S = a.ck + gh * DK * DV;
    const float* Dg = a.dl + gh * BC * DV;
    const float* Zg = a.dz + gh * BC * DV;
    const float* Ug = a.du + gh * DK * DV;

    // ---- phase 1: products over the value axis ----
    RowsIn<BC, BSV, BT3, In> rO;
    Rows<BC, BSV, BT3> rZ, rD;
    Rows<DK, BSV, BT3> rS, rU;
    Rows<BC, DK, BT3> rKh, rQt, rKt;
    auto load_slice = [&](int j0) {
        rO.load(dout + vb + j0, vst, clen);
        rZ.load(Zg + j0, DV, BC);
        rD.load(Dg + j0, DV, BC);
        rS.load(S + j0, DV, DK);
        rU.load(Ug + j0, DV, DK);
    };
    load_slice(0);
    __syncthreads();   // sgm
    for (int j0 = 0; j0 < DV; j0 += BSV) {
        rO.store(sm + OFF_O, PJ);
        rZ.store(sm + OFF_Z, PJ);
        rD.store(sm + OFF_D, PJ);
        rS.store(sm + OFF_S, PJ, sgm);   // Sm = Gm (.) S
        rU.store(sm + OFF_U, PJ);
        __syncthreads();
        if (j0 + BSV < DV) {
            load_slice(j0 + BSV);
        } else {
            rKh.load(a.kh + gh * BC * DK, DK, BC);
            rQt.load(a.qt + gh * BC * DK, DK, BC);
            rKt.load(a.kt + gh * BC * DK, DK, BC);
        }
#pragma unroll
        for (int kb2 = 0; kb2 < BSV / 16; ++kb2) {
            const float4 ao = frag4(sm + OFF_O, PJ, 16 * rt, 16 * kb2, l);
            const float4 az = frag4(sm + OFF_Z, PJ, 16 * rt, 16 * kb2, l);
            const float4 ad = frag4(sm + OFF_D, PJ, 16 * rt, 16 * kb2, l);
#pragma unroll
            for (int ct = 0; ct < NCH; ++ct) {
                const float4 bs = frag4(sm + OFF_S, PJ, ctile(ct), 16 * kb2, l);
                const float4 bu = frag4(sm + OFF_U, PJ, ctile(ct), 16 * kb2, l);
                R1[ct] = mma4x(ao, bs, R1[ct]);
                R2[ct] = mma4x(az, bs, R2[ct]);
                R3[ct] = mma4x(ad, bu, R3[ct]);
            }
            if (ch <= rt) {
                const float4 bd = frag4(sm + OFF_D, PJ, 16 * ch, 16 * kb2, l);
                dPa = mma4x(ao, bd, dPa);
                dAa = mma4x(az, bd, dAa);
            }
        }
        __syncthreads();
    }
    // ---- phase 2 ----
    {
        float* sP = sm + OFF_P;
        float* sA = sm + OFF_A;
        // dP = tril(dO Delta^T), dA = -strictly_lower(dZ Delta^T)
        if (ch <= rt) {
            const int s2 = 16 * ch + ln;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = 16 * rt + 4 * g4 + jj;
                sP[r * PC + s2] = s2 <= r ? dPa[jj] : 0.f;
                sA[r * PC + s2] = s2 < r ? -dAa[jj] : 0.f;
            }
        }
        rKh.store(sm + OFF_KH, PE);
        rQt.store(sm + OFF_QT, PE);
        rKt.store(sm + OFF_KT, PE);
#pragma unroll
        for (int ct = 0; ct < NCH; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) R2[ct][jj] = -R2[ct][jj];
        __syncthreads();
        // dQt' = R1 + dP Kh', dKt' = -R2 + dA Kh': s-blocks 0 .. rt
        for (int sb = 0; sb <= rt; ++sb) {
            const float4 ap = frag4(sP, PC, 16 * rt, 16 * sb, l);
            const float4 aa = frag4(sA, PC, 16 * rt, 16 * sb, l);
#pragma unroll
            for (int ct = 0; ct < NCH; ++ct) {
                const float4 bk = frag_col(sm + OFF_KH, PE, 16 * sb, ctile(ct), l);
                R1[ct] = mma4x(ap, bk, R1[ct]);
                R2[ct] = mma4x(aa, bk, R2[ct]);
            }
        }
        // dKh' = R3 + dP^T Qt' + dA^T Kt': r-blocks rt .. 3
        for (int rb = rt; rb < BC / 16; ++rb) {
            const float4 ap = frag_col(sP, PC, 16 * rb, 16 * rt, l);
            const float4 aa = frag_col(sA, PC, 16 * rb, 16 * rt, l);
#pragma unroll
            for (int ct = 0; ct < NCH; ++ct) {
                const float4 bq = frag_col(sm + OFF_QT, PE, 16 * rb, ctile(ct), l);
                const float4 bt = frag_col(sm + OFF_KT, PE, 16 * rb, ctile(ct), l);
                R3[ct] = mma4x(ap, bq, R3[ct]);
                R3[ct] = mma4x(aa, bt, R3[ct]);
            }
        }
    }
    // ---- epilogue ----
    // thread: channel i, rows r0 .. r0 + RPT - 1 (on one side of the
    // midpoint).  Its loads go out before the barrier: q, k, b of its rows
    // and the alphas between its rows and the midpoint (1 past the chunk).
    const int i = t % DK, rg = t / DK, r0 = RPT * rg;
    // loads unconditional (absent rows read row 0) and widened after all
    // of them are out
    RawEl<In> rq[RPT], rk[RPT], rbk[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int r = r0 + u;
        const size_t o = kb + (size_t)(r < clen ? r : 0) * kst + i;
        rq[u] = ld_raw1(q + o);
        rk[u] = ld_raw1(k + o);
        rbk[u] = ld_raw1(b + o);
    }
    RunFactors<RPT> rf;
    rf.load(alpha, kb + i, kst, r0, clen);
    float xq[RPT], xk[RPT], xb[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const bool ok = r0 + u < clen;
        xq[u] = ok ? widen1(rq[u]) : 0.f;
        xk[u] = ok ? widen1(rk[u]) : 0.f;
        xb[u] = ok ? widen1(rbk[u]) : 0.f;
    }
    float cS = 0.f, cC = 0.f;
    for (int sl = 0; sl < DV / 16; ++sl) {
        cS += a.cf[((gh * (DV / 16) + sl) * 2 + 0) * DK + i];
        cC += a.cf[((gh * (DV / 16) + sl) * 2 + 1) * DK + i];
    }
    __syncthreads();   // phase 2 done with the tiles
    float* sDQT = sm;
    float* sDKT = sm + DK * PC;
    float* sDHT = sm + 2 * DK * PC;
    float* sSum = sm + OFF_SUM;
#pragma unroll
    for (int ct = 0; ct < NCH; ++ct) {
        const int o = (ctile(ct) + ln) * PC + 16 * rt + 4 * g4;
        *reinterpret_cast<float4*>(sDQT + o) = make_float4(R1[ct][0], R1[ct][1], R1[ct][2], R1[ct][3]);
        *reinterpret_cast<float4*>(sDKT + o) = make_float4(R2[ct][0], R2[ct][1], R2[ct][2], R2[ct][3]);
        *reinterpret_cast<float4*>(sDHT + o) = make_float4(R3[ct][0], R3[ct][1], R3[ct][2], R3[ct][3]);
    }
    rf.factors(r0);   // decay factors of the thread's rows, as the prep kernel forms them
    const float* e1 = rf.e1;
    __syncthreads();
    // dq = dQt' e1; db = dKt' k e1; dk = dKt' b e1 + dKh' / e1; and
    // e = dKt' Kt' + dQt' Qt' - dKh' Kh' with the tiles formed as in prep
    float ev[RPT];
    float esum = 0.f;
    {
        Gt* gq = static_cast<Gt*>(a.dq);
        Gt* gk = static_cast<Gt*>(a.dk);
        Gt* gb = static_cast<Gt*>(a.db);
#pragma unroll
        for (int u4 = 0; u4 < RPT; u4 += 4) {
            const float4 vq = *reinterpret_cast<const float4*>(sDQT + i * PC + r0 + u4);
            const float4 vt = *reinterpret_cast<const float4*>(sDKT + i * PC + r0 + u4);
            const float4 vh = *reinterpret_cast<const float4*>(sDHT + i * PC + r0 + u4);
            const float dqt[4] = {vq.x, vq.y, vq.z, vq.w};
            const float dkt[4] = {vt.x, vt.y, vt.z, vt.w};
            const float dkh[4] = {vh.x, vh.y, vh.z, vh.w};
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int u = u4 + z, r = r0 + u;
                const float f = e1[u];
                const float kt = xb[u] * xk[u] * f, qt = xq[u] * f, kh = xk[u] / f;
                ev[u] = dkt[z] * kt + dqt[z] * qt - dkh[z] * kh;
                esum += ev[u];
                if (r < clen) {
                    const size_t o = kb + (size_t)r * kst + i;
                    store1(gq + o, dqt[z] * f);
                    store1(gb + o, dkt[z] * xk[u] * f);
                    store1(gk + o, dkt[z] * xb[u] * f + dkh[z] / f);
                }
            }
        }
    }
    sSum[rg * DK + i] = esum;
    __syncthreads();
    // dalpha_r = sum_{s >= r} e_s + [r <= mid] (cS - cC - sum_s e_s) + cC,
    // divided by alpha_r
    {
        float later = 0.f, tot = 0.f;
#pragma unroll
        for (int x = 0; x < RG; ++x) {
            const float v = sSum[x * DK + i];
            tot += v;
            later += x > rg ? v : 0.f;
        }
        const float cm = cS - cC - tot;
        Gt* ga = static_cast<Gt*>(a.dalpha);
        float suf = later;
#pragma unroll
        for (int u = RPT - 1; u >= 0; --u) {
            const int r = r0 + u;
            suf += ev[u];
            if (r < clen) {
                const float dl = suf + (r <= BMID ? cm : 0.f) + cC;
                store1(ga + kb + (size_t)r * kst + i, dl / rf.own[u]);
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
    L.nsl = dv / DSV;
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
    L.cf = o;     o += al256(u * (dv / 16) * 2 * dk * 4);
    L.total = o;
    return L;
}

template <typename In, typename Gt, int DK, int DV>
hipError_t launch_bwd_t(const BwdArgs& a, int64_t slots, hipStream_t stream) {
    const dim3 gchunks((unsigned)slots, (unsigned)a.H);
    hipLaunchKernelGGL((bwd_prep_kernel<In, DK, DV>), gchunks, dim3(BT3), 0, stream, a);
    // slabs of one (sequence, head) on one XCD: groups of 8 units
    const unsigned groups = (unsigned)((a.N * a.H + 7) / 8);
    hipLaunchKernelGGL((bwd_dstate_kernel<In, Gt, DK, DV>), dim3(groups * 8 * a.nsl), dim3(DT),
                       0, stream, a);
    hipLaunchKernelGGL((bwd_grad_kernel<In, Gt, DK, DV>), gchunks, dim3(BT3), 0, stream, a);
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
