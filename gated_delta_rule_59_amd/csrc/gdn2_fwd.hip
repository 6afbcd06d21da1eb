// gdn2_fwd.hip -- chunkwise-WY forward of the Gated Delta Rule-2 (gfx950).
//
// Method (Gated DeltaNet-2 pages: Spanish blog "Innovaciones Tecnicas" item 1;
// Korean summary "main contributions" item 3 and "method" steps 3-4): the
// sequence is cut into chunks of C = 64 tokens and the per-channel decay is
// absorbed into asymmetric erase factors.  Inside a chunk that starts from
// state S0, with g_r = sum_{s<=r} log2 alpha_s (per key channel) and
// gamma_r = 2^g_r:
//
//   Kt_r = gamma_r (.) b_r (.) k_r      Kh_s = k_s / gamma_s
//   A_rs = Kt_r . Kh_s  (s < r)         T = (I + A)^-1        X_r = w_r (.) v_r
//   W = T Kt,  U = T X,  Delta = U - W S0
//   O = Qt S0 + tril(Qt Kh^T) Delta     Qt_r = gamma_r (.) q_r
//   S_C = Diag(gamma_C) S0 + Ke^T Delta Ke_s = k_s (.) gamma_C / gamma_s
//
// which is the token recurrence rearranged exactly (no approximation).  In the
// A and tril(Qt Kh^T) products both factors are taken relative to the decay
// at the chunk midpoint, so each factor stays within 2^(half-chunk decay).
//
// Kernel design (one launch): a workgroup of 4 waves owns one (sequence,
// head, 64-column value slab) and walks that sequence's chunks in order.  The
// fp32 state slab (dk x 64) lives in MFMA accumulator registers, 16 value
// columns per wave; value columns of S never interact, so slabs of one head
// are independent workgroups.  Per chunk:
//   1. load q, k, alpha, b (dk side) and v, w (slab), in-chunk cumulative
//      log2-decay (wave shuffles + one LDS exchange), build the decayed
//      operand tiles in LDS (fp16 for bf16 inputs, fp32 for fp32 inputs);
//   2. A and P = tril(Qt' Kh'^T) on MFMA;
//   3. T = (I + A)^-1: 16x16 diagonal blocks by substitution (VALU),
//      off-diagonal blocks by MFMA, one block column per wave;
//   4. W = T Kt (shared) and U = T X (own columns) on MFMA;
//   5. per wave, with its state columns as the B operand straight from the
//      accumulators: Delta = U - W S, O = Qt S + P Delta,
//      S <- Diag(gamma_C) S + Ke^T Delta;  O is staged in LDS and stored
//      with 128-byte row segments.
// The contraction index of the products whose B operand comes from
// accumulators is permuted to match the accumulator layout; the A operand is
// read from LDS with the same permutation.
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

namespace gdn2 {

constexpr int FWD_C = 64;        // chunk length
constexpr int FWD_SV = 64;       // value columns per workgroup
constexpr int FWD_THREADS = 256; // 4 waves; wave w owns value columns 16w..16w+15

template <typename In> struct OpOf;
template <> struct OpOf<bf16_t> { using type = _Float16; };
template <> struct OpOf<float> { using type = float; };

template <typename Op> struct OpTraits;
template <> struct OpTraits<_Float16> {
    static constexpr int KSTEP = 32;  // contraction per MFMA (16x16x32 f16)
    static constexpr int PAD = 8;     // LDS row padding, elements (16 bytes)
};
template <> struct OpTraits<float> {
    static constexpr int KSTEP = 4;   // 16x16x4 f32
    static constexpr int PAD = 4;
};

// ---------------------------------------------------------------------------
// fragment helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// acc += A[16 x K] * B[K x 16] with both operands in LDS, contraction index
// contiguous: A row (a_row + (l&15)), B column (b_row + (l&15)) of a [*][pitch]
// array whose rows are the contraction index runs.  k in [k0, k0 + nk*KSTEP).
__device__ __forceinline__ floatx4 mma_ll(floatx4 acc, const _Float16* A, int apitch, int a_row,
                                          const _Float16* B, int bpitch, int b_row, int k0,
                                          int nk) {
    const int l = lane_id();
    const _Float16* pa = A + (a_row + (l & 15)) * apitch + k0 + 8 * (l >> 4);
    const _Float16* pb = B + (b_row + (l & 15)) * bpitch + k0 + 8 * (l >> 4);
    for (int s = 0; s < nk; ++s)
        acc = mma16(*reinterpret_cast<const halfx8*>(pa + 32 * s),
                    *reinterpret_cast<const halfx8*>(pb + 32 * s), acc);
    return acc;
}
__device__ __forceinline__ floatx4 mma_ll(floatx4 acc, const float* A, int apitch, int a_row,
                                          const float* B, int bpitch, int b_row, int k0, int nk) {
    const int l = lane_id();
    const float* pa = A + (a_row + (l & 15)) * apitch + k0 + (l >> 4);
    const float* pb = B + (b_row + (l & 15)) * bpitch + k0 + (l >> 4);
    for (int s = 0; s < nk; ++s) acc = mma16(pa[4 * s], pb[4 * s], acc);
    return acc;
}

// B operands held in registers, built from accumulator tiles (16 rows each).
// fp16: one halfx8 per 32 contraction rows = {tile 2m rows 4g..4g+3, tile 2m+1
// rows 4g..4g+3}.  fp32: the accumulator values themselves.
template <typename Op, int NT> struct RegB;
template <int NT> struct RegB<_Float16, NT> {
    halfx8 f[NT / 2];
    __device__ __forceinline__ void build(const floatx4* t) {
#pragma unroll
        for (int m = 0; m < NT / 2; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[m][j] = (_Float16)t[2 * m][j];
                f[m][4 + j] = (_Float16)t[2 * m + 1][j];
            }
    }
};
template <int NT> struct RegB<float, NT> {
    floatx4 f[NT];
    __device__ __forceinline__ void build(const floatx4* t) {
#pragma unroll
        for (int m = 0; m < NT; ++m) f[m] = t[m];
    }
};

// acc += A[16 x 16*ntile] * B where B comes from accumulator tiles
// 0..ntile-1 (RegB) and A is read from LDS (row a_row + (l&15), contraction
// columns k0 ...) with the matching permutation.  ntile must be even for fp16.
template <int NT>
__device__ __forceinline__ floatx4 mma_lr(floatx4 acc, const _Float16* A, int apitch, int a_row,
                                          int k0, const RegB<_Float16, NT>& B, int ntile) {
    const int l = lane_id();
    const _Float16* pa = A + (a_row + (l & 15)) * apitch + k0 + 4 * (l >> 4);
#pragma unroll
    for (int m = 0; m < NT / 2; ++m) {
        if (2 * m >= ntile) break;
        const halfx4 lo = *reinterpret_cast<const halfx4*>(pa + 32 * m);
        const halfx4 hi = *reinterpret_cast<const halfx4*>(pa + 32 * m + 16);
        halfx8 a;
        a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
        a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
        acc = mma16(a, B.f[m], acc);
    }
    return acc;
}
template <int NT>
__device__ __forceinline__ floatx4 mma_lr(floatx4 acc, const float* A, int apitch, int a_row,
                                          int k0, const RegB<float, NT>& B, int ntile) {
    const int l = lane_id();
    const float* pa = A + (a_row + (l & 15)) * apitch + k0 + 4 * (l >> 4);
#pragma unroll
    for (int m = 0; m < NT; ++m) {
        if (m >= ntile) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mma16(pa[16 * m + j], B.f[m][j], acc);
    }
    return acc;
}

// 16x16x16 product for the block inverse: A (16x16) from an LDS array whose
// rows are contiguous in the contraction index (lane reads row (l&15),
// columns 4g..4g+3 -- matching the accumulator layout of B), B an
// accumulator tile.
__device__ __forceinline__ floatx4 mma_blk(floatx4 acc, const float* A, int apitch, int a_row,
                                           int a_col, floatx4 B) {
    const int l = lane_id();
    const float* pa = A + (a_row + (l & 15)) * apitch + a_col + 4 * (l >> 4);
    halfx4 a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) { a[j] = (_Float16)pa[j]; b[j] = (_Float16)B[j]; }
    return mma16(a, b, acc);
}
__device__ __forceinline__ floatx4 mma_blk(floatx4 acc, const _Float16* A, int apitch, int a_row,
                                           int a_col, floatx4 B) {
    const int l = lane_id();
    const _Float16* pa = A + (a_row + (l & 15)) * apitch + a_col + 4 * (l >> 4);
    const halfx4 a = *reinterpret_cast<const halfx4*>(pa);
    halfx4 b;
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = (_Float16)B[j];
    return mma16(a, b, acc);
}
// fp32 variants (fp32 operand path): four 16x16x4 steps, contraction index
// 4g + j in step j.
__device__ __forceinline__ floatx4 mma_blk32(floatx4 acc, const float* A, int apitch, int a_row,
                                             int a_col, floatx4 B) {
    const int l = lane_id();
    const float* pa = A + (a_row + (l & 15)) * apitch + a_col + 4 * (l >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mma16(pa[j], B[j], acc);
    return acc;
}
template <typename Op, typename AT>
__device__ __forceinline__ floatx4 blk_mma(floatx4 acc, const AT* A, int apitch, int a_row,
                                           int a_col, floatx4 B) {
    if constexpr (sizeof(Op) == 2) return mma_blk(acc, A, apitch, a_row, a_col, B);
    else return mma_blk32(acc, A, apitch, a_row, a_col, B);
}

// Off-diagonal blocks of block column J of T = (I + A)^-1 (16x16 blocks):
// T_iJ = -T_ii sum_{m=J}^{i-1} A_im T_mJ, computed by one wave from its own
// accumulator tiles and written to sT.
template <typename Op, int J, int PA, int PC>
__device__ __forceinline__ void inverse_block_column(const float* sA, Op* sT) {
    const int l = lane_id();
    const int g4 = l >> 4, ln = l & 15;
    floatx4 Tc[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) Tc[J][jj] = (float)sT[(16 * J + 4 * g4 + jj) * PC + 16 * J + ln];
#pragma unroll
    for (int i = J + 1; i < 4; ++i) {
        floatx4 X = zero4();
#pragma unroll
        for (int m = J; m < i; ++m) X = blk_mma<Op>(X, sA, PA, 16 * i, 16 * m, Tc[m]);
        const floatx4 Y = blk_mma<Op>(zero4(), sT, PC, 16 * i, 16 * i, X);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            Tc[i][jj] = -Y[jj];
            sT[(16 * i + 4 * g4 + jj) * PC + 16 * J + ln] = (Op)(-Y[jj]);
        }
    }
}

// ---------------------------------------------------------------------------
// the fused forward kernel
// ---------------------------------------------------------------------------
template <typename In, typename Out, int DK>
__global__ __launch_bounds__(FWD_THREADS, 1) void fwd_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const In* __restrict__ alpha, const In* __restrict__ b, const In* __restrict__ w,
    const float* __restrict__ S0, Out* __restrict__ o, float* __restrict__ S_T,
    const int32_t* __restrict__ cu_seqlens, int num_pairs, int nslab, int T, int H, int DV) {
    using Op = typename OpOf<In>::type;
    constexpr int C = FWD_C;
    constexpr int SV = FWD_SV;
    constexpr int KSTEP = OpTraits<Op>::KSTEP;
    constexpr int PK = DK + OpTraits<Op>::PAD;  // pitch of [C][DK] tiles
    constexpr int PC = C + OpTraits<Op>::PAD;   // pitch of [*][C] tiles
    constexpr int PA = C + 1;                   // pitch of the fp32 A tile
    constexpr int NST = DK / 16;                // state accumulator tiles per wave
    constexpr int CGK = DK / 8;                 // 8-channel groups across dk
    constexpr int RPTK = C * CGK / FWD_THREADS; // consecutive rows per thread (dk side)
    constexpr int RGW = 64 / CGK;               // row groups per wave (dk side)

    // ---- workgroup -> (pair, slab); slabs of one pair share an XCD ----
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int slab = (bid >> 3) % nslab;
    const int pair = (bid / (8 * nslab)) * 8 + xcd;
    if (pair >= num_pairs) return;
    const int n = pair / H;
    const int h = pair - n * H;
    int64_t row0, len;
    if (cu_seqlens) {
        row0 = cu_seqlens[n];
        len = (int64_t)cu_seqlens[n + 1] - row0;
    } else {
        row0 = (int64_t)n * T;
        len = T;
    }

    // LDS regions (bytes); W, T and the O staging reuse tiles that are dead by then
    constexpr int TILE_K = C * PK * (int)sizeof(Op);   // [C][DK] operand tile
    constexpr int TILE_T = DK * PC * (int)sizeof(Op);  // [DK][C] transposed tile
    constexpr int OFF_KT = 0;                          // Kt' (mid-referenced); then -W
    constexpr int OFF_KH = OFF_KT + TILE_K;            // Kh'
    constexpr int OFF_Q2 = OFF_KH + TILE_K;            // Qt'; then T
    constexpr int OFF_Q = OFF_Q2 + TILE_K;             // Qt
    constexpr int OFF_KTT = OFF_Q + TILE_K;            // Kt^T
    constexpr int OFF_KET = OFF_KTT + TILE_T;          // Ke^T
    constexpr int OFF_XT = OFF_KET + TILE_T;           // X^T (own slab)
    constexpr int OFF_P = OFF_XT + SV * PC * (int)sizeof(Op);  // P = tril(Qt' Kh'^T)
    constexpr int OFF_A = OFF_P + C * PC * (int)sizeof(Op);    // A (fp32)
    constexpr int OFF_TOT = OFF_A + C * PA * 4;        // per-wave log2-decay totals [4][DK]
    constexpr int OFF_GC = OFF_TOT + 4 * DK * 4;       // gamma_C [DK]
    constexpr int END0 = OFF_GC + DK * 4;
    constexpr bool O_IN_KH = TILE_K >= C * SV * 4;     // fp32 O staging fits over Kh'
    constexpr int OFF_O = O_IN_KH ? OFF_KH : (END0 + 15) / 16 * 16;
    constexpr int LDS_BYTES = O_IN_KH ? END0 : OFF_O + C * SV * 4;
    static_assert(C * PC <= C * PK, "T must fit over Qt'");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __align__(16) unsigned char smem[LDS_BYTES];
    Op* const sKt = reinterpret_cast<Op*>(smem + OFF_KT);
    Op* const sKh = reinterpret_cast<Op*>(smem + OFF_KH);
    Op* const sQ2 = reinterpret_cast<Op*>(smem + OFF_Q2);
    Op* const sQ = reinterpret_cast<Op*>(smem + OFF_Q);
    Op* const sKtT = reinterpret_cast<Op*>(smem + OFF_KTT);
    Op* const sKeT = reinterpret_cast<Op*>(smem + OFF_KET);
    Op* const sXT = reinterpret_cast<Op*>(smem + OFF_XT);
    Op* const sP = reinterpret_cast<Op*>(smem + OFF_P);
    float* const sA = reinterpret_cast<float*>(smem + OFF_A);
    float (*const sTot)[DK] = reinterpret_cast<float (*)[DK]>(smem + OFF_TOT);
    float* const sGamC = reinterpret_cast<float*>(smem + OFF_GC);
    Op* const sW = sKt;
    Op* const sT = sQ2;
    float* const sO = reinterpret_cast<float*>(smem + OFF_O);

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int wave = tid >> 6;
    const int g4 = l >> 4;   // lane group
    const int ln = l & 15;   // lane column
    const int vcol0 = slab * SV + 16 * wave;  // first value column of this wave

    // upper-triangle tiles of P that the PDelta product reads stay zero
    for (int e = tid; e < C * PC; e += FWD_THREADS) {
        const int r = e / PC, c = e % PC;
        if (c >= C || (c >> 4) > (r >> 4)) sP[e] = (Op)0.f;
    }

    // ---- state slab into accumulators: wave owns columns vcol0..vcol0+15 ----
    floatx4 Sacc[NST];
    {
        const float* sp = S0 ? S0 + (size_t)pair * DK * DV + vcol0 + ln : nullptr;
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                Sacc[t][j] = sp ? sp[(size_t)(16 * t + 4 * g4 + j) * DV] : 0.f;
    }

    const int cg = tid % CGK;          // dk-side channel group (channels 8cg..8cg+7)
    const int rgk = tid / CGK;         // dk-side row group (rows rgk*RPTK ..)
    const int cgv = tid & 7;           // slab-side channel group
    const int rgv = tid >> 3;          // slab-side rows 2rgv, 2rgv+1
    const size_t kstride = (size_t)H * DK;
    const size_t vstride = (size_t)H * DV;

    const int64_t nchunks = (len + C - 1) / C;
    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t c0 = ci * C;
        const int clen = (int)((len - c0) < C ? (len - c0) : C);

        // ---------------- 1. loads, cumulative log2 decay, operand tiles ------
        float gq[RPTK][8], gk[RPTK][8], gb[RPTK][8], gl[RPTK][8];
#pragma unroll
        for (int m = 0; m < RPTK; ++m) {
            const int r = rgk * RPTK + m;
            if (r < clen) {
                const size_t off = (size_t)(row0 + c0 + r) * kstride + (size_t)h * DK + 8 * cg;
                load8(q + off, gq[m]);
                load8(k + off, gk[m]);
                load8(b + off, gb[m]);
                load8(alpha + off, gl[m]);
#pragma unroll
                for (int i = 0; i < 8; ++i) gl[m][i] = log2f(gl[m][i]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) { gq[m][i] = 0.f; gk[m][i] = 0.f; gb[m][i] = 0.f; gl[m][i] = 0.f; }
            }
        }
        float xv[2][8];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int r = 2 * rgv + m;
            if (r < clen) {
                const size_t off = (size_t)(row0 + c0 + r) * vstride + (size_t)h * DV + slab * SV + 8 * cgv;
                float vv[8], ww[8];
                load8(v + off, vv);
                load8(w + off, ww);
#pragma unroll
                for (int i = 0; i < 8; ++i) xv[m][i] = ww[i] * vv[i];
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) xv[m][i] = 0.f;
            }
        }
        // inclusive cumsum over the thread's rows, then over the wave's row groups
#pragma unroll
        for (int m = 1; m < RPTK; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i) gl[m][i] += gl[m - 1][i];
        float tot[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) tot[i] = gl[RPTK - 1][i];
        float pre[8];
        const int rgl = rgk % RGW;  // row group within the wave
        {
            float inc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) inc[i] = tot[i];
#pragma unroll
            for (int d = 1; d < RGW; d <<= 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float up = __shfl_up(inc[i], d * CGK);
                    if (rgl >= d) inc[i] += up;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) pre[i] = inc[i] - tot[i];  // exclusive prefix in wave
            if (rgl == RGW - 1)
#pragma unroll
                for (int i = 0; i < 8; ++i) sTot[wave][8 * cg + i] = inc[i];
        }
        __syncthreads();
        float gmid[8], gC[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int ch = 8 * cg + i;
            const float t0 = sTot[0][ch], t1 = sTot[1][ch], t2 = sTot[2][ch], t3 = sTot[3][ch];
            float wpre = 0.f;
            if (wave >= 1) wpre += t0;
            if (wave >= 2) wpre += t1;
            if (wave >= 3) wpre += t2;
            pre[i] += wpre;
            gmid[i] = t0 + t1;
            gC[i] = t0 + t1 + t2 + t3;
        }
        if (wave == 0 && rgl == 0)
#pragma unroll
            for (int i = 0; i < 8; ++i) sGamC[8 * cg + i] = exp2f(gC[i]);
        // decayed operand tiles
        {
            float em[8], eCm[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) { em[i] = exp2f(gmid[i]); eCm[i] = exp2f(gC[i] - gmid[i]); }
            Op tKt[RPTK][8], tKe[RPTK][8];
#pragma unroll
            for (int m = 0; m < RPTK; ++m) {
                const int r = rgk * RPTK + m;
                Op a1[8], a2[8], a3[8], a4[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float g = gl[m][i] + pre[i];
                    const float e1 = exp2f(g - gmid[i]);
                    const float e1i = exp2f(gmid[i] - g);
                    const float bk = gb[m][i] * gk[m][i];
                    a1[i] = (Op)(bk * e1);                 // Kt'
                    a2[i] = (Op)(gk[m][i] * e1i);          // Kh'
                    a3[i] = (Op)(gq[m][i] * e1);           // Qt'
                    a4[i] = (Op)(gq[m][i] * (e1 * em[i])); // Qt
                    tKt[m][i] = (Op)(bk * (e1 * em[i]));   // Kt
                    tKe[m][i] = (Op)(gk[m][i] * (e1i * eCm[i]));  // Ke
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    sKt[r * PK + 8 * cg + i] = a1[i];
                    sKh[r * PK + 8 * cg + i] = a2[i];
                    sQ2[r * PK + 8 * cg + i] = a3[i];
                    sQ[r * PK + 8 * cg + i] = a4[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int m = 0; m < RPTK; ++m) {
                    sKtT[(8 * cg + i) * PC + rgk * RPTK + m] = tKt[m][i];
                    sKeT[(8 * cg + i) * PC + rgk * RPTK + m] = tKe[m][i];
                }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int m = 0; m < 2; ++m) sXT[(8 * cgv + i) * PC + 2 * rgv + m] = (Op)xv[m][i];
        }
        __syncthreads();

        // ---------------- 2. A = strictly_lower(Kt' Kh'^T), P = tril(Qt' Kh'^T) ----
        for (int job = wave; job < 20; job += 4) {
            const int isP = job >= 10;
            const int t = isP ? job - 10 : job;
            // (R, S) pairs in order (0,0),(1,0),(1,1),(2,0),(2,1),(2,2),(3,0)..(3,3)
            const int R = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
            const int Sb = t - (R * (R + 1)) / 2;
            floatx4 acc = zero4();
            acc = mma_ll(acc, isP ? sQ2 : sKt, PK, 16 * R, sKh, PK, 16 * Sb, 0, DK / KSTEP);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * R + 4 * g4 + j;
                const int c = 16 * Sb + ln;
                if (isP) sP[r * PC + c] = (Op)(r >= c ? acc[j] : 0.f);
                else sA[r * PA + c] = r > c ? acc[j] : 0.f;
            }
        }
        __syncthreads();

        // ---------------- 3. T = (I + A)^-1 -----------------------------------
        // 3a. diagonal 16x16 blocks by forward substitution, lane = column
        if (ln == l) {  // lanes 0..15 of every wave; wave w inverts block w
            const int base = 16 * wave;
            float col[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = (r == ln) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) x -= sA[(base + r) * PA + base + s] * col[s];
                col[r] = x;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[(base + r) * PC + base + ln] = (Op)col[r];
        }
        // tiles (0,1) and (2,3) lie inside the 32-wide contraction steps of W/U
        if (wave == 0 || wave == 2) {
            const int R = wave, Sb = wave + 1;
            for (int e = l; e < 256; e += 64)
                sT[(16 * R + (e >> 4)) * PC + 16 * Sb + (e & 15)] = (Op)0.f;
        }
        __syncthreads();
        // 3b. block column j = wave (0..2): T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj
        if (wave == 0) inverse_block_column<Op, 0, PA, PC>(sA, sT);
        else if (wave == 1) inverse_block_column<Op, 1, PA, PC>(sA, sT);
        else if (wave == 2) inverse_block_column<Op, 2, PA, PC>(sA, sT);
        __syncthreads();

        // ---------------- 4. W = T Kt (shared), U = T X (own columns) ------------
        {
            constexpr int NCT = DK / 16;  // column tiles of W
            for (int ct = wave; ct < NCT; ct += 4) {
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    const int nk = (16 * R + 16 + KSTEP - 1) / KSTEP;
                    floatx4 acc = zero4();
                    acc = mma_ll(acc, sT, PC, 16 * R, sKtT, PC, 16 * ct, 0, nk);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        sW[(16 * R + 4 * g4 + jj) * PK + 16 * ct + ln] = (Op)(-acc[jj]);
                }
            }
        }
        floatx4 D[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            const int nk = (16 * R + 16 + KSTEP - 1) / KSTEP;
            D[R] = mma_ll(zero4(), sT, PC, 16 * R, sXT, PC, 16 * wave, 0, nk);
        }
        __syncthreads();

        // ---------------- 5. per-wave value side ---------------------------------
        RegB<Op, NST> SB;
        SB.build(Sacc);
#pragma unroll
        for (int R = 0; R < 4; ++R) D[R] = mma_lr(D[R], sW, PK, 16 * R, 0, SB, NST);  // U - W S
        RegB<Op, 4> DB;
        DB.build(D);
        floatx4 O[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            O[R] = mma_lr(zero4(), sQ, PK, 16 * R, 0, SB, NST);                       // Qt S
            const int nt = (sizeof(Op) == 2) ? ((R >> 1) + 1) * 2 : R + 1;
            O[R] = mma_lr(O[R], sP, PC, 16 * R, 0, DB, nt);                           // + P Delta
        }
#pragma unroll
        for (int t = 0; t < NST; ++t) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) Sacc[t][jj] *= sGamC[16 * t + 4 * g4 + jj];
            Sacc[t] = mma_lr(Sacc[t], sKeT, PC, 16 * t, 0, DB, 4);                   // + Ke^T Delta
        }
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sO[(16 * R + 4 * g4 + jj) * SV + 16 * wave + ln] = O[R][jj];
        __syncthreads();
        {
            const int r = tid >> 2;
            const int cb = (tid & 3) * 16;
            if (r < clen) {
                Out* dst = o + (size_t)(row0 + c0 + r) * vstride + (size_t)h * DV + slab * SV + cb;
                const float* src = sO + r * SV + cb;
#pragma unroll
                for (int e = 0; e < 16; e += 4) store4(dst + e, src[e], src[e + 1], src[e + 2], src[e + 3]);
            }
        }
        // the next chunk's first LDS writes follow its cumsum barrier
    }

    if (S_T) {
        float* sp = S_T + (size_t)pair * DK * DV + vcol0 + ln;
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) sp[(size_t)(16 * t + 4 * g4 + j) * DV] = Sacc[t][j];
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
FwdPlan plan_fwd(int B, int T, int H, int dk, int dv, int num_seqs, int in_dtype) {
    (void)B; (void)T; (void)H; (void)dk; (void)num_seqs; (void)in_dtype;
    FwdPlan p;
    p.nslab = dv / FWD_SV;
    p.workspace = 0;
    return p;
}

template <typename In, typename Out, int DK>
static hipError_t launch_fwd_t(const FwdPlan& plan, const void* q, const void* k, const void* v,
                               const void* alpha, const void* b, const void* w, const float* S0,
                               void* o, float* S_T, const int32_t* cu, int N, int T, int H,
                               int dv, hipStream_t stream) {
    const int num_pairs = N * H;
    const int groups = (num_pairs + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * plan.nslab));
    hipLaunchKernelGGL((fwd_kernel<In, Out, DK>), grid, dim3(FWD_THREADS), 0, stream,
                       static_cast<const In*>(q), static_cast<const In*>(k),
                       static_cast<const In*>(v), static_cast<const In*>(alpha),
                       static_cast<const In*>(b), static_cast<const In*>(w), S0,
                       static_cast<Out*>(o), S_T, cu, num_pairs, plan.nslab, T, H, dv);
    return hipGetLastError();
}

template <typename In, typename Out>
static hipError_t launch_fwd_dk(const FwdPlan& plan, const void* q, const void* k, const void* v,
                                const void* alpha, const void* b, const void* w, const float* S0,
                                void* o, float* S_T, const int32_t* cu, int N, int T, int H, int dk,
                                int dv, hipStream_t stream) {
    // fp32 operand tiles for dk = 128 would need 253 KB of LDS (160 KB limit)
    if constexpr (sizeof(typename OpOf<In>::type) == 2) {
        if (dk == 128)
            return launch_fwd_t<In, Out, 128>(plan, q, k, v, alpha, b, w, S0, o, S_T, cu, N, T, H,
                                              dv, stream);
    }
    if (dk != 64) return hipErrorInvalidValue;
    return launch_fwd_t<In, Out, 64>(plan, q, k, v, alpha, b, w, S0, o, S_T, cu, N, T, H, dv, stream);
}

hipError_t launch_fwd(const FwdPlan& plan, const void* q, const void* k, const void* v,
                      const void* alpha, const void* b, const void* w, int in_dtype,
                      const float* S0, void* o, int out_dtype, float* S_T,
                      const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int dk,
                      int dv, void* workspace, hipStream_t stream) {
    (void)workspace;
    const int N = cu_seqlens ? num_seqs : B;
    if (N == 0 || ((int64_t)B * T == 0 && S_T == nullptr)) return hipSuccess;  // nothing to do
    if (in_dtype == DT_BF16) {
        if (out_dtype == DT_BF16)
            return launch_fwd_dk<bf16_t, bf16_t>(plan, q, k, v, alpha, b, w, S0, o, S_T,
                                                 cu_seqlens, N, T, H, dk, dv, stream);
        return launch_fwd_dk<bf16_t, float>(plan, q, k, v, alpha, b, w, S0, o, S_T, cu_seqlens, N,
                                            T, H, dk, dv, stream);
    }
    return launch_fwd_dk<float, float>(plan, q, k, v, alpha, b, w, S0, o, S_T, cu_seqlens, N, T,
                                       H, dk, dv, stream);
}

}  // namespace gdn2
