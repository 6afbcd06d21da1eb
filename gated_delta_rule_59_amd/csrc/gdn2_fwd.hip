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
// Kernels (one launch per forward, plus two more for long sequences):
//  - fwd_ws_kernel, bf16 inputs: a workgroup of 8 waves owns one (sequence or
//    segment, head, 64-column value slab) and walks its chunks in order.
//    Value waves 0-3 hold the fp32 state slab in MFMA accumulator registers
//    (16 columns each) and run the state step; key waves 4-7 build the next
//    chunk's decayed fp16 operand tiles in LDS meanwhile.  Two barriers per
//    chunk: step M (state step of chunk c || tiles of chunk c+1), then step 2
//    (A, P and the inverses of A's 16x16 diagonal blocks for chunk c+1).
//    Delta comes from block forward substitution with those inverses; T, W
//    and U are never formed.  A chunk whose half-chunk decay leaves the fp16
//    range sends its sequence to a token-serial fp32 redo in the same launch.
//  - fwd_kernel, fp32 inputs (dk = 64): a workgroup of 4 waves runs, per
//    chunk, one phase per barrier: operand tiles (fp32); A and P on MFMA;
//    T = (I + A)^-1 by diagonal blocks and MFMA; W = T Kt and U = T X; the
//    state step Delta = U - W S, O = Qt S + P Delta, S <- Diag(gamma_C) S +
//    Ke^T Delta.
//  - Long sequences with few (sequence, head) pairs: a summary pass composes
//    each segment's affine map of the state, seg_combine_kernel chains the
//    maps, and the forward pass runs every segment from its start state.
//  - Gate forms (Spanish blog "Jerarquia de Generalizacion"; Japanese article
//    "core"): b, w (Kimi Delta Attention form) and alpha (Gated DeltaNet
//    form) may come as one value per (token, head).  fwd_ws_kernel is compiled
//    per form and widens such a value to the channels right after its load;
//    fwd_kernel reads the form at run time.
// The contraction index of the products whose B operand comes from
// accumulators is permuted to match the accumulator layout; the A operand is
// read from LDS with the same permutation.
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

#include <type_traits>

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
// With SWAP the MFMA operands are exchanged, which yields the transposed
// tile: the lane then holds row a_row + (l&15), columns b_row + 4g .. 4g+3.
template <bool SWAP = false>
__device__ __forceinline__ floatx4 mma_ll(floatx4 acc, const _Float16* A, int apitch, int a_row,
                                          const _Float16* B, int bpitch, int b_row, int k0,
                                          int nk) {
    const int l = lane_id();
    const _Float16* pa = A + (a_row + (l & 15)) * apitch + k0 + 8 * (l >> 4);
    const _Float16* pb = B + (b_row + (l & 15)) * bpitch + k0 + 8 * (l >> 4);
    for (int s = 0; s < nk; ++s) {
        const halfx8 fa = *reinterpret_cast<const halfx8*>(pa + 32 * s);
        const halfx8 fb = *reinterpret_cast<const halfx8*>(pb + 32 * s);
        acc = SWAP ? mma16(fb, fa, acc) : mma16(fa, fb, acc);
    }
    return acc;
}
template <bool SWAP = false>
__device__ __forceinline__ floatx4 mma_ll(floatx4 acc, const float* A, int apitch, int a_row,
                                          const float* B, int bpitch, int b_row, int k0, int nk) {
    const int l = lane_id();
    const float* pa = A + (a_row + (l & 15)) * apitch + k0 + (l >> 4);
    const float* pb = B + (b_row + (l & 15)) * bpitch + k0 + (l >> 4);
    for (int s = 0; s < nk; ++s)
        acc = SWAP ? mma16(pb[4 * s], pa[4 * s], acc) : mma16(pa[4 * s], pb[4 * s], acc);
    return acc;
}

// Transposed tiles ([channel][token], 64 tokens per row) are stored with the
// 8-element block index of each row XORed with (row >> 4) & 7: the writers
// (4 consecutive tokens of channels 8 apart) then hit distinct LDS banks,
// while a 16-row fragment read keeps one key for all its rows.
__device__ __forceinline__ int swz(int row, int col) { return col ^ (((row >> 4) & 7) << 3); }
// The Kh'^T tile of the wave-specialised forward uses the same key with its
// bits placed differently: key bit 0 flips column bit 5 (the 32-column
// half), bits 1 and 2 flip column bits 3 and 4.  Its writers (4 channel rows
// 8 apart, 32 tokens each, per 32 lanes) then cover all 64 banks, while a
// 16-row read still sees one key.
__device__ __forceinline__ int swz_kh(int row, int col) {
    const int k = (row >> 4) & 7;
    return col ^ (((k & 1) << 5) | (((k >> 1) & 1) << 3) | (((k >> 2) & 1) << 4));
}

// fp16 operand tiles whose contraction index meets a B operand built from
// accumulator tiles store their columns permuted within each 32-column block:
// logical column 32m + 16h + 4g + j sits at 32m + 8g + 4h + j.  The 8 values
// lane group g needs for one 16x16x32 step ({4g..4g+3, 16+4g..16+4g+3}) are
// then one aligned 16-byte LDS read.  Products whose two operands both come
// from such tiles see the same permutation on both sides, which leaves the
// contraction unchanged.
__device__ __forceinline__ int pcol(int c) {
    return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}

// As mma_ll, with the B operand in a swizzled transposed tile (k0 = 0).
template <bool SWAP = false>
__device__ __forceinline__ floatx4 mma_ls(floatx4 acc, const _Float16* A, int apitch, int a_row,
                                          const _Float16* B, int bpitch, int b_row, int nk) {
    const int l = lane_id();
    const int brow = b_row + (l & 15);
    const _Float16* pa = A + (a_row + (l & 15)) * apitch + 8 * (l >> 4);
    const _Float16* pb = B + brow * bpitch;
    for (int s = 0; s < nk; ++s) {
        const halfx8 fa = *reinterpret_cast<const halfx8*>(pa + 32 * s);
        const halfx8 fb = *reinterpret_cast<const halfx8*>(pb + swz(brow, 8 * (l >> 4) + 32 * s));
        acc = SWAP ? mma16(fb, fa, acc) : mma16(fa, fb, acc);
    }
    return acc;
}
template <bool SWAP = false>
__device__ __forceinline__ floatx4 mma_ls(floatx4 acc, const float* A, int apitch, int a_row,
                                          const float* B, int bpitch, int b_row, int nk) {
    const int l = lane_id();
    const int brow = b_row + (l & 15);
    const float* pa = A + (a_row + (l & 15)) * apitch + (l >> 4);
    const float* pb = B + brow * bpitch;
    for (int s = 0; s < nk; ++s) {
        const float fa = pa[4 * s], fb = pb[swz(brow, (l >> 4) + 4 * s)];
        acc = SWAP ? mma16(fb, fa, acc) : mma16(fa, fb, acc);
    }
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
    // the same from tiles holding the negated values
    __device__ __forceinline__ void build_neg(const floatx4* t) {
#pragma unroll
        for (int m = 0; m < NT / 2; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[m][j] = (_Float16)(-t[2 * m][j]);
                f[m][4 + j] = (_Float16)(-t[2 * m + 1][j]);
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

// fp32 operand path: acc += A[16 x 16*ntile] * B where B comes from
// accumulator tiles 0..ntile-1 (RegB) and A is read from LDS (row
// a_row + (l&15), contraction columns k0 ...) in the accumulator order: step j
// of tile m contracts index 16m + 4g + j.  With SWAP the MFMA operands are
// exchanged: the register tiles act as the transposed left factor and the
// result is (A . B)^T, i.e. the lane holds row a_row + (l&15) of A . B at
// columns 4g .. 4g+3.
template <bool SWAP, int NT>
__device__ __forceinline__ floatx4 mma_lr_(floatx4 acc, const float* A, int apitch, int a_row,
                                           int k0, const RegB<float, NT>& B, int ntile) {
    const int l = lane_id();
    const float* pa = A + (a_row + (l & 15)) * apitch + k0 + 4 * (l >> 4);
#pragma unroll
    for (int m = 0; m < NT; ++m) {
        if (m >= ntile) break;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = SWAP ? mma16(B.f[m][j], pa[16 * m + j], acc) : mma16(pa[16 * m + j], B.f[m][j], acc);
    }
    return acc;
}
template <typename Op, int NT>
__device__ __forceinline__ floatx4 mma_lr(floatx4 acc, const Op* A, int apitch, int a_row, int k0,
                                          const RegB<Op, NT>& B, int ntile) {
    return mma_lr_<false>(acc, A, apitch, a_row, k0, B, ntile);
}
// (A . B)^T tile with B from registers: lane holds (A.B)[a_row + (l&15)][4g .. 4g+3]
template <typename Op, int NT>
__device__ __forceinline__ floatx4 mma_rl(floatx4 acc, const RegB<Op, NT>& B, int ntile,
                                          const Op* A, int apitch, int a_row) {
    return mma_lr_<true>(acc, A, apitch, a_row, 0, B, ntile);
}

// As mma_lr, with the A operand in a swizzled transposed tile (k0 = 0).
template <int NT>
__device__ __forceinline__ floatx4 mma_lrs(floatx4 acc, const float* A, int apitch, int a_row,
                                           const RegB<float, NT>& B, int ntile) {
    const int l = lane_id();
    const int arow = a_row + (l & 15);
    const float* pa = A + arow * apitch;
#pragma unroll
    for (int m = 0; m < NT; ++m) {
        if (m >= ntile) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mma16(pa[swz(arow, 16 * m + 4 * (l >> 4) + j)], B.f[m][j], acc);
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
                                           int a_col, floatx4 B, int l = lane_id()) {
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
                                           int a_col, floatx4 B, int l = lane_id()) {
    if constexpr (sizeof(Op) == 2) return mma_blk(acc, A, apitch, a_row, a_col, B, l);
    else return mma_blk32(acc, A, apitch, a_row, a_col, B);
}

// C + X Y for 16x16 blocks given as accumulator tiles of X^T and of Y (the
// accumulator layout of X^T is the A-operand layout of X).
template <typename Op>
__device__ __forceinline__ floatx4 prod16(floatx4 XtAcc, floatx4 YAcc, floatx4 C) {
    if constexpr (sizeof(Op) == 2) {
        halfx4 a, b;
#pragma unroll
        for (int j = 0; j < 4; ++j) { a[j] = (_Float16)XtAcc[j]; b[j] = (_Float16)YAcc[j]; }
        return mma16(a, b, C);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) C = mma16(XtAcc[j], YAcc[j], C);
        return C;
    }
}

// (I + N)^-1 of a 16x16 diagonal block, N strictly lower (so N^16 = 0), given
// as the accumulator tiles of N and N^T: (I - N)(I + N^2)(I + N^4)(I + N^8).
// Returns the accumulator tile: lane holds T[4g + j][(l&15)].
template <typename Op>
__device__ __forceinline__ floatx4 diag_block_inverse(floatx4 N, floatx4 Nt, int l = lane_id()) {
    const int g4 = l >> 4, ln = l & 15;
    const floatx4 z = zero4();
    const floatx4 N2 = prod16<Op>(Nt, N, z);     // N N
    const floatx4 N2t = prod16<Op>(N, Nt, z);    // N^T N^T
    const floatx4 N4 = prod16<Op>(N2t, N2, z);
    const floatx4 N4t = prod16<Op>(N2, N2t, z);
    const floatx4 N8t = prod16<Op>(N4, N4t, z);
    floatx4 Z;
#pragma unroll
    for (int j = 0; j < 4; ++j) Z[j] = ((4 * g4 + j == ln) ? 1.f : 0.f) - N[j];
    Z = prod16<Op>(N2t, Z, Z);                   // (I + N^2) Z
    Z = prod16<Op>(N4t, Z, Z);                   // (I + N^4) Z
    Z = prod16<Op>(N8t, Z, Z);                   // (I + N^8) Z
    return Z;
}

// 4 consecutive elements of one row, from an accumulator holding them
__device__ __forceinline__ void st4(_Float16* p, floatx4 x) {
    halfx4 h;
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = (_Float16)x[j];
    *reinterpret_cast<halfx4*>(p) = h;
}
__device__ __forceinline__ void st4(float* p, floatx4 x) { *reinterpret_cast<floatx4*>(p) = x; }
template <typename Op>
__device__ __forceinline__ void st_neg4(Op* p, floatx4 x) { st4(p, -x); }

// Off-diagonal blocks of block column J of T = (I + A)^-1 (16x16 blocks):
// T_iJ = -T_ii sum_{m=J}^{i-1} A_im T_mJ, computed by one wave from its own
// accumulator tiles and written to sT.
template <typename Op, int J, int PA, int PC, typename AT>
__device__ __forceinline__ void inverse_block_column(const AT* sA, Op* sT, floatx4 Tjj,
                                                     int l = lane_id()) {
    const int g4 = l >> 4, ln = l & 15;
    floatx4 Tc[4];
    Tc[J] = Tjj;
#pragma unroll
    for (int i = J + 1; i < 4; ++i) {
        floatx4 X = zero4();
#pragma unroll
        for (int m = J; m < i; ++m) X = blk_mma<Op>(X, sA, PA, 16 * i, 16 * m, Tc[m], l);
        const floatx4 Y = blk_mma<Op>(zero4(), sT, PC, 16 * i, 16 * i, X, l);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            Tc[i][jj] = -Y[jj];
            sT[(16 * i + 4 * g4 + jj) * PC + 16 * J + ln] = (Op)(-Y[jj]);
        }
    }
}


// ---------------------------------------------------------------------------
// raw chunk inputs held in registers (prefetched one chunk ahead)
// ---------------------------------------------------------------------------
template <typename In> struct Raw8;
template <> struct Raw8<bf16_t> {
    u16x8 v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const u16x8*>(p); }
    // one value per (token, head), broadcast over the 8 channels
    __device__ __forceinline__ void load_bcast(const bf16_t* p) {
        const uint16_t u = p->bits;
        v = u16x8{u, u, u, u, u, u, u, u};
    }
    __device__ __forceinline__ void widen(float (&x)[8]) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = bf16_to_f32(v[i]);
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void load_bcast(const float* p) {
        const float x = *p;
        a = make_float4(x, x, x, x);
        b = a;
    }
    __device__ __forceinline__ void widen(float (&x)[8]) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};
template <typename In, int RPTK> struct ChunkRaw {
    Raw8<In> q[RPTK], k[RPTK], b[RPTK], a[RPTK];  // dk side: RPTK consecutive rows, 8 channels
    Raw8<In> v[2], w[2];                          // value slab: 2 consecutive rows, 8 channels
};

// vector LDS stores of 8 consecutive row elements / RPTK consecutive column elements
__device__ __forceinline__ void st_row8(_Float16* p, const float (&x)[8]) {
    halfx8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)x[i];
    *reinterpret_cast<halfx8*>(p) = h;
}
__device__ __forceinline__ void st_row8(float* p, const float (&x)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
template <int N> __device__ __forceinline__ void st_col(_Float16* p, const float* x) {
    if constexpr (N == 4) {
        halfx4 h;
        h[0] = (_Float16)x[0]; h[1] = (_Float16)x[1]; h[2] = (_Float16)x[2]; h[3] = (_Float16)x[3];
        *reinterpret_cast<halfx4*>(p) = h;
    } else {
        static_assert(N == 2, "column run");
        halfx2 h;
        h[0] = (_Float16)x[0]; h[1] = (_Float16)x[1];
        *reinterpret_cast<halfx2*>(p) = h;
    }
}
template <int N> __device__ __forceinline__ void st_col(float* p, const float* x) {
    if constexpr (N == 4) *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    else *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
}
// physical column of logical contraction column c: permuted for fp16 tiles,
// plain for fp32 tiles (whose 16x16x4 steps read single elements)
template <typename Op> __device__ __forceinline__ int opcol(int c) {
    if constexpr (sizeof(Op) == 2) return pcol(c);
    else return c;
}
// logical columns c0 .. c0+7 (c0 a multiple of 8) of one tile row
__device__ __forceinline__ void st_row8p(_Float16* row, int c0, const float (&x)[8]) {
    halfx4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) { lo[i] = (_Float16)x[i]; hi[i] = (_Float16)x[4 + i]; }
    *reinterpret_cast<halfx4*>(row + pcol(c0)) = lo;
    *reinterpret_cast<halfx4*>(row + pcol(c0 + 4)) = hi;
}
__device__ __forceinline__ void st_row8p(float* row, int c0, const float (&x)[8]) { st_row8(row + c0, x); }

// x from the lane SH positions lower in the same 16-lane row, or 1 where
// that lane is outside the row (DPP row_shr with the update kept at `old`)
template <int SH>
__device__ __forceinline__ float dpp_shr_or1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x),
                                                      0x110 + SH, 0xF, 0xF, false));
}

// ---- explicit fp16 fragment loads (row row0 + (l&15) of a [*][pitch] tile) ----
// contraction columns 32s + 8g .. +7
__device__ __forceinline__ halfx8 ld_std(const _Float16* A, int pitch, int row0, int s,
                                         int l = lane_id()) {
    return *reinterpret_cast<const halfx8*>(A + (row0 + (l & 15)) * pitch + 32 * s + 8 * (l >> 4));
}
__device__ __forceinline__ halfx8 ld_std_swz(const _Float16* A, int pitch, int row0, int s,
                                             int l = lane_id()) {
    const int row = row0 + (l & 15);
    return *reinterpret_cast<const halfx8*>(A + row * pitch + swz(row, 32 * s + 8 * (l >> 4)));
}
// Buffer descriptor over `bytes` bytes from p (raw buffer: offsets are
// range-checked against `bytes`, reads out of range return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ floatx4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// the same with the non-temporal hint (cache policy bit 1), for data read
// once by one workgroup: v and w of a value slab.  (The dk-side inputs are
// read by every slab workgroup of a head through one L2: they keep the
// default policy; non-temporal loads there made the 1.3B-layer launch 9%
// slower.)
__device__ __forceinline__ floatx4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
// one 16-bit element, in the low half of element 0
__device__ __forceinline__ floatx4 buf_ld2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const uint32_t u = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
    x[0] = __uint_as_float(u);
    return x;
}
// 4 consecutive outputs at byte offset off (the whole offset in the VGPR
// operand, which the range check covers): stores past the range are dropped
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, const floatx4& x,
                                        const float*) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, const floatx4& x,
                                        const bf16_t*) {
    const u32x2_t d = {f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3])};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, (int)off, 0, 0);
}
// The [C][DK] operand tiles of the wave-specialised forward (Kt', Qt') have
// pitch DK + 16 halves, and row r has the 8-column blocks of its permuted
// columns swapped in pairs when bit 2 of r is set.  Fragment reads (16
// consecutive rows, 16 bytes per lane) and the key waves' row stores (4
// rows 4 apart, 8 bytes per lane) then both spread over the LDS banks.
__device__ __forceinline__ int swz_kq(int row, int col) { return col ^ (((row >> 2) & 1) << 3); }
// fragment of rows 16R .. 16R+15: the lane's block is 32s + 8(g ^ bit 2 of its row)
__device__ __forceinline__ halfx8 ld_std_kq(const _Float16* A, int pitch, int R, int s, int l) {
    const int ln = l & 15;
    return *reinterpret_cast<const halfx8*>(A + (16 * R + ln) * pitch + 32 * s +
                                            8 * ((l >> 4) ^ ((ln >> 2) & 1)));
}
// logical columns c0 .. c0+7 (c0 a multiple of 8) of row r
__device__ __forceinline__ void st_row8kq(_Float16* tile, int pitch, int r, int c0,
                                          const float (&x)[8]) {
    halfx4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) { lo[i] = (_Float16)x[i]; hi[i] = (_Float16)x[4 + i]; }
    _Float16* row = tile + r * pitch;
    *reinterpret_cast<halfx4*>(row + swz_kq(r, pcol(c0))) = lo;
    *reinterpret_cast<halfx4*>(row + swz_kq(r, pcol(c0 + 4))) = hi;
}

// ---- products with lanes SH positions lower in the same 16-lane DPP row,
// 8 independent values ----
// The compiler's hazard checks do not look inside inline assembly, so each
// block starts with two wait states (a DPP source written by the previous
// VALU instruction needs them) and interleaves the 8 values, so that no DPP
// instruction reads a register written by either of the two before it.
// Lanes whose DPP source lies outside the row are not written and keep the
// destination's old value.
#define GDN2_DPPMUL(D, S, K) \
    "v_mul_f32_dpp %" #D ", %" #S ", %" #D " row_shr:%c" #K " row_mask:0xf bank_mask:0xf\n\t"
// x <- x(lane - SH) * x; lanes (l & 15) < SH keep x
template <int SH>
__device__ __forceinline__ void dpp_shr_mul8(float (&x)[8]) {
    asm("s_nop 1\n\t"
        GDN2_DPPMUL(0, 0, 8) GDN2_DPPMUL(1, 1, 8) GDN2_DPPMUL(2, 2, 8) GDN2_DPPMUL(3, 3, 8)
        GDN2_DPPMUL(4, 4, 8) GDN2_DPPMUL(5, 5, 8) GDN2_DPPMUL(6, 6, 8) GDN2_DPPMUL(7, 7, 8)
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
          "+v"(x[7])
        : "i"(SH));
}
// y <- x(lane - SH) * y; lanes (l & 15) < SH keep y
template <int SH>
__device__ __forceinline__ void dpp_shr_mul8_into(const float (&x)[8], float (&y)[8]) {
    asm("s_nop 1\n\t"
        GDN2_DPPMUL(0, 8, 16) GDN2_DPPMUL(1, 9, 16) GDN2_DPPMUL(2, 10, 16) GDN2_DPPMUL(3, 11, 16)
        GDN2_DPPMUL(4, 12, 16) GDN2_DPPMUL(5, 13, 16) GDN2_DPPMUL(6, 14, 16) GDN2_DPPMUL(7, 15, 16)
        : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]),
          "+v"(y[7])
        : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]),
          "i"(SH));
}
// x <- x(lane - SH mod 16, same row) * x: every lane is written
template <int SH>
__device__ __forceinline__ void dpp_ror_mul8(float (&x)[8]) {
#define GDN2_RORMUL(D) \
    "v_mul_f32_dpp %" #D ", %" #D ", %" #D " row_ror:%c8 row_mask:0xf bank_mask:0xf\n\t"
    asm("s_nop 1\n\t"
        GDN2_RORMUL(0) GDN2_RORMUL(1) GDN2_RORMUL(2) GDN2_RORMUL(3)
        GDN2_RORMUL(4) GDN2_RORMUL(5) GDN2_RORMUL(6) GDN2_RORMUL(7)
        : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
          "+v"(x[7])
        : "i"(SH));
#undef GDN2_RORMUL
}
#undef GDN2_DPPMUL
// A = strictly_lower(Kt' Kh'^T) and P = tril(Qt' Kh'^T): 10 lower 16x16 tiles
// each, five jobs per wave.  Job 0 of wave W is the diagonal A tile (W, W): it
// is returned in registers in both orientations (accumulator tiles of N and
// N^T, strictly lower part kept) for the block inverse and not stored.
struct ApJob { bool isP; int R, S; };
template <int W, int J>
__device__ __forceinline__ constexpr ApJob ap_job() {
    // A00 A10 A20 P00 P30 | A11 A21 A30 P10 P31 | A22 A31 P11 P20 P32 | A33 A32 P21 P22 P33
    constexpr ApJob t[4][5] = {
        {{false, 0, 0}, {false, 1, 0}, {false, 2, 0}, {true, 0, 0}, {true, 3, 0}},
        {{false, 1, 1}, {false, 2, 1}, {false, 3, 0}, {true, 1, 0}, {true, 3, 1}},
        {{false, 2, 2}, {false, 3, 1}, {true, 1, 1}, {true, 2, 0}, {true, 3, 2}},
        {{false, 3, 3}, {false, 3, 2}, {true, 2, 1}, {true, 2, 2}, {true, 3, 3}}};
    return t[W][J];
}

template <typename Op, int DK, int PK, int PC, int PA, int W, bool WITH_P>
__device__ __forceinline__ void ap_tiles(const Op* sKt, const Op* sKh, const Op* sQ2, Op* sP,
                                         float* sA, floatx4& N, floatx4& Nt) {
    constexpr int KSTEP = OpTraits<Op>::KSTEP;
    const int l = lane_id();
    const int g4 = l >> 4, ln = l & 15;
    floatx4 acc[5];
    floatx4 accN;  // diagonal tile in the untransposed orientation
#define GDN2_JOB(J) constexpr ApJob jb##J = ap_job<W, J>();
    GDN2_JOB(0) GDN2_JOB(1) GDN2_JOB(2) GDN2_JOB(3) GDN2_JOB(4)
#undef GDN2_JOB
    constexpr ApJob jobs[5] = {jb0, jb1, jb2, jb3, jb4};
    if constexpr (sizeof(Op) == 2) {
        // contraction step outer, jobs inner: independent accumulators
#pragma unroll
        for (int jn = 0; jn < 5; ++jn) acc[jn] = zero4();
        accN = zero4();
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
            halfx8 fa[5], fb[5];
#pragma unroll
            for (int jn = 0; jn < 5; ++jn) {
                if (!WITH_P && jobs[jn].isP) continue;
                fa[jn] = ld_std(jobs[jn].isP ? sQ2 : sKt, PK, 16 * jobs[jn].R, s);
                fb[jn] = ld_std(sKh, PK, 16 * jobs[jn].S, s);
            }
            // transposed products: lane holds row 16R + (l&15), columns 16S + 4g .. 4g+3
#pragma unroll
            for (int jn = 0; jn < 5; ++jn)
                if (WITH_P || !jobs[jn].isP) acc[jn] = mma16(fb[jn], fa[jn], acc[jn]);
            accN = mma16(fa[0], fb[0], accN);
        }
    } else {
#pragma unroll
        for (int jn = 0; jn < 5; ++jn)
            if (WITH_P || !jobs[jn].isP)
                acc[jn] = mma_ll<true>(zero4(), jobs[jn].isP ? sQ2 : sKt, PK, 16 * jobs[jn].R, sKh,
                                       PK, 16 * jobs[jn].S, 0, DK / KSTEP);
        accN = mma_ll<false>(zero4(), sKt, PK, 16 * W, sKh, PK, 16 * W, 0, DK / KSTEP);
    }
    // diagonal block: N[4g+j][ln] in accN, N^T[4g+j][ln] = N[ln][4g+j] in acc[0]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        N[j] = (4 * g4 + j > ln) ? accN[j] : 0.f;
        Nt[j] = (ln > 4 * g4 + j) ? acc[0][j] : 0.f;
    }
#pragma unroll
    for (int jn = 1; jn < 5; ++jn) {
        if (!WITH_P && jobs[jn].isP) continue;
        const int r = 16 * jobs[jn].R + ln;
        floatx4 x = acc[jn];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 16 * jobs[jn].S + 4 * g4 + j;
            if (jobs[jn].isP ? (r < c) : (r <= c)) x[j] = 0.f;
        }
        if (jobs[jn].isP) st4(sP + r * PC + opcol<Op>(16 * jobs[jn].S + 4 * g4), x);
        else st4(sA + r * PA + 16 * jobs[jn].S + 4 * g4, x);
    }
}

// ---------------------------------------------------------------------------
// the fused forward kernel
// ---------------------------------------------------------------------------
// Workgroup -> work unit.  Workgroups are dealt to the 8 XCDs round-robin
// (blockIdx.x & 7), and the nsl value slabs of a unit are consecutive
// workgroups of one XCD, so they share that XCD's L2.
//  - Dense batches: each XCD receives a contiguous block of units; with the
//    [B, T, H, d] layout the units of one sequence then share one L2, which
//    sees whole token rows (all heads) requested together.
//  - Packed batches with a length order (sequence indices, longest first):
//    the units are dealt in that order, round-robin over the XCDs, so the
//    longest sequences start first and every XCD gets a similar share.
// Returns -1 for padding workgroups.
__device__ __forceinline__ int work_unit(int units, int nsl, const int32_t* order, int H) {
    const int xcd = blockIdx.x & 7;
    const int j = (blockIdx.x >> 3) / nsl;
    const int per_xcd = (units + 7) / 8;
    if (j >= per_xcd) return -1;
    if (order) {
        const int rank = j * 8 + xcd;
        if (rank >= units) return -1;
        return order[rank / H] * H + rank % H;
    }
    const int unit = xcd * per_xcd + j;
    return unit < units ? unit : -1;
}

// Launch arguments of fwd_kernel.
struct FwdArgs {
    const void *q, *k, *v, *alpha, *b, *w;
    const float* S0;      // [N, H, dk, dv] or null (zeros)
    void* o;              // [B, T, H, dv]
    float* S_T;           // [N, H, dk, dv] or null
    const int32_t* cu_seqlens;
    int num_pairs;        // N * H
    int nslab;            // value slabs (dv / 64)
    int T, H, DV;
    // Long sequences are split into nseg segments of seg_chunks chunks (no
    // varlen).  MODE_SUMMARY composes each segment's affine map of the state,
    // S_end = M S_start + H, into maps[pair][seg][dk][dv + dk] ([H | M]): the
    // dk columns of M run as nslab_m extra slabs with X = 0 and an identity
    // start.  MODE_FWD then runs every segment from its start state
    // (starts[pair][seg][dk][dv] for seg >= 1, S0 for seg 0).
    int nseg, seg_chunks, nslab_m;
    float* maps;
    const float* starts;
    // packed batches: sequence indices by decreasing length, or null
    const int32_t* order;
    // MODE_CKPT: chunk start states and final states (ckpt_slot0)
    float* ckpt;
    // gate shapes (GATES_*): b, w and for GATES_GDN alpha may hold one value
    // per (token, head), [rows, H], broadcast over their channels
    int gates;
};
enum { MODE_FWD = 0, MODE_SUMMARY = 1, MODE_CKPT = 2 };

// Stores a wave's 16 state columns (accumulator layout: ST[t][j] = S[16t +
// 4g + j][vcol0 + ln]) into checkpoint slot `slot` of head h.
template <int DK>
__device__ __forceinline__ void store_ckpt(float* ckpt, int64_t slot, int H, int h, int DV,
                                           int vcol0, const floatx4 (&ST)[DK / 16]) {
    const int l = threadIdx.x & 63, g4 = l >> 4, ln = l & 15;
    float* p = ckpt + ((size_t)slot * H + h) * DK * DV + vcol0 + ln;
#pragma unroll
    for (int t = 0; t < DK / 16; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[(size_t)(16 * t + 4 * g4 + j) * DV] = ST[t][j];
}

// Rows of segment `seg` of sequence n (dense: batch row n; packed: tokens
// cu_seqlens[n] ..), and how many segments that sequence has.  Segments are
// seg_chunks chunks long; a packed batch reserves nseg slots per sequence (the
// longest possible) and a workgroup past its sequence's count has no work.
__device__ __forceinline__ void seg_rows(const FwdArgs& a, int n, int seg, int64_t& row0,
                                         int64_t& len, int& nseg_n) {
    int64_t start, L;
    if (a.cu_seqlens) {
        start = a.cu_seqlens[n];
        L = (int64_t)a.cu_seqlens[n + 1] - start;
    } else {
        start = (int64_t)n * a.T;
        L = a.T;
    }
    if (a.nseg == 1) {
        row0 = start;
        len = L;
        nseg_n = 1;
        return;
    }
    const int64_t seg_rows_n = (int64_t)a.seg_chunks * FWD_C;
    const int64_t nch = (L + FWD_C - 1) / FWD_C;
    nseg_n = nch <= 0 ? 1 : (int)((nch + a.seg_chunks - 1) / a.seg_chunks);
    const int64_t s0 = (int64_t)seg * seg_rows_n;
    row0 = start + s0;
    len = L - s0 < seg_rows_n ? L - s0 : seg_rows_n;
    if (len < 0) len = 0;
}

// ---- 4 consecutive storage elements widened to fp32 ----
__device__ __forceinline__ void load4f(const bf16_t* p, float (&x)[4]) {
    const u16x4 u = *reinterpret_cast<const u16x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = bf16_to_f32(u[j]);
}
__device__ __forceinline__ void load4f(const float* p, float (&x)[4]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
}

// Token-serial path of the chunked kernels, for a sequence (segment) whose
// chunks left the range of the chunked operands: the decode step per token in
// fp32 on one wave's 16 value columns, with the state in the chunked kernels'
// accumulator layout (ST[t][j] = S[16t + 4g + j][vcol0 + ln], lane = 16g + ln,
// already reset to the start state).  Row sums go over the lane's DK/4 rows,
// then across the four lane groups by lane swaps.  aph / bph: alpha / b and w
// given per (token, head).  Writes o (unless summary) for every token of the
// sequence (segment); M slabs (mslab) run with X = 0.  With ckpt, stores the
// state at every 64th token into checkpoint slots slot, slot + 1, ...
template <typename In, typename Out, int DK>
__device__ __forceinline__ void token_serial_redo(floatx4 (&ST)[DK / 16], const FwdArgs& a,
                                                  bool aph, bool bph, bool summary, bool mslab,
                                                  int64_t row0, int64_t len, int h, int vcol0,
                                                  float* ckpt = nullptr, int64_t slot = 0) {
    constexpr int NST = DK / 16;
    const In* __restrict__ q = static_cast<const In*>(a.q);
    const In* __restrict__ k = static_cast<const In*>(a.k);
    const In* __restrict__ v = static_cast<const In*>(a.v);
    const In* __restrict__ alpha = static_cast<const In*>(a.alpha);
    const In* __restrict__ b = static_cast<const In*>(a.b);
    const In* __restrict__ w = static_cast<const In*>(a.w);
    Out* __restrict__ o = static_cast<Out*>(a.o);
    const int H = a.H, DV = a.DV;
    const int l = threadIdx.x & 63, g4 = l >> 4, ln = l & 15;
    for (int64_t tt = 0; tt < len; ++tt) {
        // checkpoint mode: the state at every chunk start
        if (ckpt && (tt & 63) == 0) store_ckpt<DK>(ckpt, slot + tt / 64, H, h, DV, vcol0, ST);
        const size_t th = (size_t)(row0 + tt) * H + h;   // per-(token, head) gates
        const size_t kb = th * DK + 4 * g4;
        float r = 0.f, p = 0.f, qk = 0.f;
        float kr[NST][4];
        const float ga = aph ? load1(alpha + th) : 0.f, gb = bph ? load1(b + th) : 0.f;
#pragma unroll
        for (int t = 0; t < NST; ++t) {
            float fa[4], fb[4], fq[4], fk[4];
            if (aph) { fa[0] = fa[1] = fa[2] = fa[3] = ga; }
            else load4f(alpha + kb + 16 * t, fa);
            if (bph) { fb[0] = fb[1] = fb[2] = fb[3] = gb; }
            else load4f(b + kb + 16 * t, fb);
            load4f(q + kb + 16 * t, fq);
            load4f(k + kb + 16 * t, fk);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kr[t][j] = fk[j];
                ST[t][j] *= fa[j];
                r += fb[j] * fk[j] * ST[t][j];
                p += fq[j] * ST[t][j];
                qk += fq[j] * fk[j];
            }
        }
        r = sum_over_rows16(r);
        p = sum_over_rows16(p);
        qk = sum_over_rows16(qk);
        const size_t vb = th * DV + vcol0 + ln;
        const float x = mslab ? 0.f : load1(w + (bph ? th : vb)) * load1(v + vb);
        const float d = x - r;   // delta of column ln
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) ST[t][j] += kr[t][j] * d;
        if (!summary && g4 == 0) store1(o + vb, p + qk * d);
    }
}

template <typename In, typename Out, int DK, int MODE>
__global__ __launch_bounds__(FWD_THREADS, 1) void fwd_kernel(FwdArgs args) {
    const In* __restrict__ q = static_cast<const In*>(args.q);
    const In* __restrict__ k = static_cast<const In*>(args.k);
    const In* __restrict__ v = static_cast<const In*>(args.v);
    const In* __restrict__ alpha = static_cast<const In*>(args.alpha);
    const In* __restrict__ b = static_cast<const In*>(args.b);
    const In* __restrict__ w = static_cast<const In*>(args.w);
    Out* __restrict__ o = static_cast<Out*>(args.o);
    const int H = args.H, DV = args.DV, T = args.T;
    constexpr bool SUMMARY = MODE == MODE_SUMMARY;
    // checkpoint mode: the forward without outputs that stores every chunk's
    // start state (and the final state) for the backward
    constexpr bool CKPT = MODE == MODE_CKPT;
    constexpr bool NOQ = SUMMARY || CKPT;   // no q, P or o
    using Op = typename OpOf<In>::type;
    constexpr int C = FWD_C;
    constexpr int SV = FWD_SV;
    constexpr int KSTEP = OpTraits<Op>::KSTEP;
    constexpr int PK = DK + OpTraits<Op>::PAD;  // pitch of [C][DK] tiles
    constexpr int PC = C + OpTraits<Op>::PAD;   // pitch of [*][C] tiles
    constexpr int PA = C + 4;                   // pitch of the fp32 A tile (16-byte rows)
    constexpr int NST = DK / 16;                // state accumulator tiles per wave
    // dk side of phase 1: wave w owns key channels [w dk/4, (w+1) dk/4) over all
    // C rows, so the in-chunk decay products are scanned within the wave
    constexpr int NCG = DK / 32;                // 8-channel groups per wave
    constexpr int RPTK = NCG;                   // consecutive rows per thread
    constexpr int RGW = C / RPTK;               // row groups per wave

    // ---- workgroup -> (pair, segment, slab); slabs of one unit share an XCD ----
    const int nsl = args.nslab + (SUMMARY ? args.nslab_m : 0);
    const int nseg = args.nseg;
    const int unit = work_unit(args.num_pairs * nseg, nsl, args.order, args.H);
    if (unit < 0) return;
    const int slab = (blockIdx.x >> 3) % nsl;
    const int pair = unit / nseg;
    const int seg = unit - pair * nseg;
    const bool mslab = SUMMARY && slab >= args.nslab;  // a column block of M (X = 0)
    const int n = pair / H;
    const int h = pair - n * H;
    int64_t row0, len;
    int nseg_n;   // segments of this sequence
    seg_rows(args, n, seg, row0, len, nseg_n);
    if (seg >= nseg_n) return;                   // a packed sequence shorter than nseg slots
    if (SUMMARY && seg == nseg_n - 1) return;    // the last segment's map is never used

    // LDS regions (bytes); W, T and the O staging reuse tiles that are dead by then
    constexpr int TILE_K = C * PK * (int)sizeof(Op);   // [C][DK] operand tile
    constexpr int TILE_T = DK * PC * (int)sizeof(Op);  // [DK][C] transposed tile
    constexpr int PO = SV + 4;                         // pitch of the fp32 O staging
    constexpr int OFF_KT = 0;                          // Kt' ; then -W'
    constexpr int OFF_KH = OFF_KT + TILE_K;            // Kh'
    constexpr int OFF_Q2 = OFF_KH + TILE_K;            // Qt'
    constexpr int OFF_KTT = OFF_Q2 + TILE_K;           // Kt'^T
    constexpr int OFF_KHT = OFF_KTT + TILE_T;          // Kh'^T
    constexpr int OFF_XT = OFF_KHT + TILE_T;           // X^T (own slab)
    constexpr int OFF_P = OFF_XT + SV * PC * (int)sizeof(Op);  // P = tril(Qt' Kh'^T)
    constexpr int OFF_A = OFF_P + C * PC * (int)sizeof(Op);    // A (fp32); then O staging
    constexpr int OFF_T = OFF_A + C * PA * 4;          // T = (I + A)^-1
    constexpr int OFF_GC = OFF_T + C * PC * (int)sizeof(Op);  // gamma_C, gamma_mid, gamma_C/gamma_mid
    constexpr int OFF_RT = OFF_GC + 3 * DK * 4;        // per-wave row totals of the decay scan
    constexpr int LDS_BYTES = OFF_RT + 4 * 4 * NCG * 8 * 4;
    static_assert(C * PO <= C * PA, "O staging must fit over A");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __align__(16) unsigned char smem[LDS_BYTES];
    Op* const sKt = reinterpret_cast<Op*>(smem + OFF_KT);
    Op* const sKh = reinterpret_cast<Op*>(smem + OFF_KH);
    Op* const sQ2 = reinterpret_cast<Op*>(smem + OFF_Q2);
    Op* const sKtT = reinterpret_cast<Op*>(smem + OFF_KTT);
    Op* const sKhT = reinterpret_cast<Op*>(smem + OFF_KHT);
    Op* const sXT = reinterpret_cast<Op*>(smem + OFF_XT);
    Op* const sP = reinterpret_cast<Op*>(smem + OFF_P);
    float* const sA = reinterpret_cast<float*>(smem + OFF_A);
    float* const sGamC = reinterpret_cast<float*>(smem + OFF_GC);   // gamma_C
    float* const sGamM = sGamC + DK;                                 // gamma_mid
    float* const sGamR = sGamC + 2 * DK;                             // gamma_C / gamma_mid
    float* const sRowTot = reinterpret_cast<float*>(smem + OFF_RT);
    Op* const sW = sKt;
    Op* const sT = reinterpret_cast<Op*>(smem + OFF_T);
    float* const sO = sA;

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int wave = tid >> 6;
    const int g4 = l >> 4;   // lane group
    const int ln = l & 15;   // lane column
    const int vcol0 = slab * SV + 16 * wave;  // first value column of this wave

    // upper-triangle tiles of P and T, which the P Delta, W' and U products
    // read, stay zero: every chunk rewrites only the lower tiles
    for (int e = tid; e < C * PC; e += FWD_THREADS) {
        sP[e] = (Op)0.f;
        sT[e] = (Op)0.f;
    }

    // checkpoint mode: slot of this segment's first chunk, and of the
    // sequence's final state
    int64_t ck_slot = 0, ck_final = 0;
    if constexpr (CKPT) {
        const int64_t s0 = ckpt_slot0(args.cu_seqlens, T, n);
        ck_slot = s0 + (int64_t)seg * args.seg_chunks;
        const int64_t Ln = args.cu_seqlens ? (int64_t)args.cu_seqlens[n + 1] - args.cu_seqlens[n]
                                           : (int64_t)T;
        ck_final = s0 + (Ln + FWD_C - 1) / FWD_C;
    }
    // Set when some chunk's decay leaves the range of the fp32 factors (see
    // phase 1); the sequence (segment) is then redone token by token.
    __shared__ int s_bad;
    if (tid == 0) s_bad = 0;
    __syncthreads();

    // ---- state slab into accumulators: wave owns columns vcol0..vcol0+15 ----
    floatx4 Sacc[NST];
    auto init_state = [&]() {
        const float* sp = nullptr;
        if (!SUMMARY) {
            // segmented: every segment's start (S0 for the first) comes from
            // the combine pass, so no workgroup of this launch reads S0 while
            // another may be writing S_T over it (S_T == S0 is allowed)
            if (nseg == 1) sp = args.S0 ? args.S0 + (size_t)pair * DK * DV + vcol0 + ln : nullptr;
            else sp = args.starts + ((size_t)pair * nseg + seg) * DK * DV + vcol0 + ln;
        }
        if (sp) {
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) Sacc[t][j] = sp[(size_t)(16 * t + 4 * g4 + j) * DV];
        } else if (mslab) {
            // identity columns: M starts as I
            const int col = (slab - args.nslab) * SV + 16 * wave + ln;
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) Sacc[t][j] = (16 * t + 4 * g4 + j == col) ? 1.f : 0.f;
        } else {
#pragma unroll
            for (int t = 0; t < NST; ++t) Sacc[t] = zero4();
        }
        // settle the S0 loads here, so that no wait on them (which would also
        // wait for the in-flight prefetch) is placed inside the chunk loop
        __builtin_amdgcn_s_waitcnt(0);
    };
    init_state();

    const int cgl = l % NCG;           // channel group within the wave
    const int cg = wave * NCG + cgl;   // dk-side channel group (channels 8cg..8cg+7)
    const int rgk = l / NCG;           // dk-side row group (rows rgk*RPTK ..)
    const int cgv = tid & 7;           // slab-side channel group
    const int rgv = tid >> 3;          // slab-side rows 2rgv, 2rgv+1
    const size_t kstride = (size_t)H * DK;
    const size_t vstride = (size_t)H * DV;

    const int64_t nchunks = (len + C - 1) / C;
    ChunkRaw<In, RPTK> cur;  // reloaded in place once phase 1 has consumed it
    // Inputs of one chunk, in five parts (q, k, b, alpha, v+w) so that the
    // prefetch of the next chunk can be spread over this chunk's phases:
    // issued at once they stall the wave on the CU's outstanding-miss limit.
    // Rows past the end of the sequence are clamped to its last row (always
    // in bounds; phase 1 treats them as absent), so that every load is
    // unconditional and the loads of one part stay in flight together.
    auto load_part = [&](ChunkRaw<In, RPTK>& R, int64_t cstart, int part) {
        const int64_t rem = len - cstart;
        const int last = (int)(rem < C ? rem : C) - 1;
        if (part < 4) {
#pragma unroll
            for (int m = 0; m < RPTK; ++m) {
                const int r = min(rgk * RPTK + m, last);
                const size_t off = (size_t)(row0 + cstart + r) * kstride + (size_t)h * DK + 8 * cg;
                const size_t th = (size_t)(row0 + cstart + r) * H + h;   // per-(token, head) gate
                if (part == 0) { if (!NOQ) R.q[m].load(q + off); }
                else if (part == 1) R.k[m].load(k + off);
                else if (part == 2) {
                    if (args.gates != GATES_FULL) R.b[m].load_bcast(b + th);
                    else R.b[m].load(b + off);
                } else {
                    if (args.gates == GATES_GDN) R.a[m].load_bcast(alpha + th);
                    else R.a[m].load(alpha + off);
                }
            }
        } else if (!mslab) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int r = min(2 * rgv + m, last);
                const size_t off = (size_t)(row0 + cstart + r) * vstride + (size_t)h * DV + slab * SV + 8 * cgv;
                R.v[m].load(v + off);
                if (args.gates != GATES_FULL) R.w[m].load_bcast(w + (size_t)(row0 + cstart + r) * H + h);
                else R.w[m].load(w + off);
            }
        }
    };
    auto load_chunk = [&](ChunkRaw<In, RPTK>& R, int64_t cstart) {
#pragma unroll
        for (int part = 0; part < 5; ++part) load_part(R, cstart, part);
    };
    if (nchunks > 0) load_chunk(cur, 0);

    for (int64_t ci = 0; ci < nchunks; ++ci) {
        const int64_t c0 = ci * C;
        const int clen = (int)((len - c0) < C ? (len - c0) : C);

        // Phase 1 is instantiated twice: full chunks skip the row masks.
        auto phase1 = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        // ---------------- 1. in-chunk decay products, operand tiles -------------
        // gamma_r = prod_{s<=r} alpha_s per key channel, as running products:
        // within the thread's rows, across the wave's row groups (shuffles)
        // and across waves (one LDS exchange).
        // (rows past the end hold a copy of the last row: masked by selects,
        // without branches, so the prefetch registers are read unconditionally)
        float gp[RPTK][8];  // alpha, then the inclusive in-chunk product
#pragma unroll
        for (int m = 0; m < RPTK; ++m) {
            const bool ok = FULL || rgk * RPTK + m < clen;
            cur.a[m].widen(gp[m]);
#pragma unroll
            for (int i = 0; i < 8; ++i) gp[m][i] = ok ? gp[m][i] : 1.f;
        }
        float xv[2][8];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bool ok = !mslab && (FULL || 2 * rgv + m < clen);
            float vv[8], ww[8];
            if (!mslab) {
                cur.v[m].widen(vv);
                cur.w[m].widen(ww);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[m][i] = ok ? ww[i] * vv[i] : 0.f;
        }
#pragma unroll
        for (int m = 1; m < RPTK; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i) gp[m][i] *= gp[m - 1][i];
        float pre[8];  // product over the earlier rows of the chunk half
        float rmid[8], gmid[8], gR[8], gC[8];  // 1/gamma_mid, gamma_mid, gamma_C/gamma_mid, gamma_C
        {
            // rows of one channel group sit NCG lanes apart: scan inside each
            // 16-lane row with DPP shifts, then combine the four row totals
            // through a wave-private LDS slot (no workgroup barrier)
            float inc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) inc[i] = gp[RPTK - 1][i];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                inc[i] *= dpp_shr_or1<NCG>(inc[i]);
                if constexpr (2 * NCG < 16) inc[i] *= dpp_shr_or1<2 * NCG>(inc[i]);
                if constexpr (4 * NCG < 16) inc[i] *= dpp_shr_or1<4 * NCG>(inc[i]);
                if constexpr (8 * NCG < 16) inc[i] *= dpp_shr_or1<8 * NCG>(inc[i]);
                pre[i] = dpp_shr_or1<NCG>(inc[i]);  // exclusive within the 16-lane row
            }
            float* slot = sRowTot + wave * (4 * NCG * 8);  // [row][cgl][8]
            if ((l & 15) >= 16 - NCG) {
                float4* d = reinterpret_cast<float4*>(slot + ((l >> 4) * NCG + cgl) * 8);
                d[0] = make_float4(inc[0], inc[1], inc[2], inc[3]);
                d[1] = make_float4(inc[4], inc[5], inc[6], inc[7]);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
            __builtin_amdgcn_wave_barrier();
            float rt[4][8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float4* sp = reinterpret_cast<const float4*>(slot + (r * NCG + cgl) * 8);
                const float4 u0 = sp[0], u1 = sp[1];
                rt[r][0] = u0.x; rt[r][1] = u0.y; rt[r][2] = u0.z; rt[r][3] = u0.w;
                rt[r][4] = u1.x; rt[r][5] = u1.y; rt[r][6] = u1.z; rt[r][7] = u1.w;
            }
            // Both chunk halves are referenced to the midpoint: pre becomes
            // the product over the rows of the lane's half before its own
            // rows, so no factor carries more than half a chunk of decay.
            const int myrow = l >> 4;
            float mn = 1.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float pr = 1.f;
                if (myrow == 1) pr = rt[0][i];
                if (myrow == 3) pr = rt[2][i];
                pre[i] *= pr;
                gmid[i] = rt[0][i] * rt[1][i];           // rows 0 .. C/2-1
                gR[i] = rt[2][i] * rt[3][i];             // rows C/2 .. C-1: gamma_C/gamma_mid
                gC[i] = gmid[i] * gR[i];                 // all rows
                rmid[i] = __builtin_amdgcn_rcpf(gmid[i]);
                mn = fminf(mn, fminf(gmid[i], gR[i]));
            }
            // The fp32 factors stay finite and normal while the decay over
            // either half of the chunk is at least 2^-126 in every channel;
            // otherwise (or on a non-finite value) the sequence (segment) is
            // recomputed token by token after the chunk loop.
            if (__builtin_amdgcn_ballot_w64(!(mn >= 0x1p-126f)) != 0 && l == 0) s_bad = 1;
        }
        if (rgk == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sGamC[8 * cg + i] = gC[i];
                sGamM[8 * cg + i] = gmid[i];
                sGamR[8 * cg + i] = gR[i];
            }
        }
        // operand tiles relative to the chunk midpoint:
        //   Kt' = b k gamma_r/gamma_mid, Kh' = k gamma_mid/gamma_r, Qt' = q gamma_r/gamma_mid
        {
            float tKt[8][RPTK], tKh[8][RPTK];
#pragma unroll
            for (int m = 0; m < RPTK; ++m) {
                const int r = rgk * RPTK + m;
                float gq[8], gk[8], gb[8];
                if (!NOQ) cur.q[m].widen(gq);
                else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) gq[i] = 0.f;
                }
                cur.k[m].widen(gk);
                cur.b[m].widen(gb);
                const bool ok = FULL || r < clen;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    gq[i] = ok ? gq[i] : 0.f;
                    gk[i] = ok ? gk[i] : 0.f;
                }
                float a1[8], a2[8], a3[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    // gamma_r / gamma_mid: gamma_r times 1/gamma_mid in the
                    // first half, the product after the midpoint in the second
                    const float gr = gp[m][i] * pre[i];
                    const float e1 = (l >> 4) < 2 ? gr * rmid[i] : gr;
                    const float e1i = __builtin_amdgcn_rcpf(e1);
                    const float bk = gb[i] * gk[i];
                    a1[i] = bk * e1;
                    a2[i] = gk[i] * e1i;
                    a3[i] = gq[i] * e1;
                    tKt[i][m] = a1[i];
                    tKh[i][m] = a2[i];
                }
                st_row8p(sKt + r * PK, 8 * cg, a1);
                st_row8p(sKh + r * PK, 8 * cg, a2);
                if (!NOQ) st_row8p(sQ2 + r * PK, 8 * cg, a3);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = 8 * cg + i;
                st_col<RPTK>(sKtT + row * PC + swz(row, rgk * RPTK), tKt[i]);
                st_col<RPTK>(sKhT + row * PC + swz(row, opcol<Op>(rgk * RPTK)), tKh[i]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = 8 * cgv + i;
                const float x2[2] = {xv[0][i], xv[1][i]};
                st_col<2>(sXT + row * PC + swz(row, 2 * rgv), x2);
            }
        }
        };
        if (clen == C) phase1(std::true_type{});
        else phase1(std::false_type{});

        // the next chunk's inputs are in flight while this chunk is computed
        const bool pf = ci + 1 < nchunks;
        if (pf) load_part(cur, c0 + C, 0);
        __syncthreads();

        // ---------------- 2. A = strictly_lower(Kt' Kh'^T), P = tril(Qt' Kh'^T) ----
        //    and the 16x16 diagonal blocks of T = (I + A)^-1, one per wave, on
        //    MFMA from registers: (I - N)(I + N^2)(I + N^4)(I + N^8)
        floatx4 Tdiag;
        {
            floatx4 N, Nt;
            if (wave == 0) ap_tiles<Op, DK, PK, PC, PA, 0, !NOQ>(sKt, sKh, sQ2, sP, sA, N, Nt);
            else if (wave == 1) ap_tiles<Op, DK, PK, PC, PA, 1, !NOQ>(sKt, sKh, sQ2, sP, sA, N, Nt);
            else if (wave == 2) ap_tiles<Op, DK, PK, PC, PA, 2, !NOQ>(sKt, sKh, sQ2, sP, sA, N, Nt);
            else ap_tiles<Op, DK, PK, PC, PA, 3, !NOQ>(sKt, sKh, sQ2, sP, sA, N, Nt);
            Tdiag = diag_block_inverse<Op>(N, Nt);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                sT[(16 * wave + 4 * g4 + jj) * PC + 16 * wave + ln] = (Op)Tdiag[jj];
        }
        if (pf) load_part(cur, c0 + C, 1);
        __syncthreads();

        // ---------------- 3. off-diagonal blocks of T ----------------------------
        // block column j = wave (0..2): T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj
        if (wave == 0) inverse_block_column<Op, 0, PA, PC>(sA, sT, Tdiag);
        else if (wave == 1) inverse_block_column<Op, 1, PA, PC>(sA, sT, Tdiag);
        else if (wave == 2) inverse_block_column<Op, 2, PA, PC>(sA, sT, Tdiag);
        if (pf) load_part(cur, c0 + C, 2);
        __syncthreads();

        // ---------------- 4. W' = T Kt' (shared, stored negated), U = T X -------
        floatx4 D[4];
        if constexpr (sizeof(Op) == 2) {
            // T fragments (lower triangle only) shared by the W' and U products
            halfx8 ft[4][2];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int st = 0; st < 2; ++st)
                    if (st <= (R >> 1)) ft[R][st] = ld_std(sT, PC, 16 * R, st);
            constexpr int NCT = DK / 16;
#pragma unroll
            for (int cc = 0; cc < NCT / 4; ++cc) {
                const int ct = wave + 4 * cc;
                const halfx8 fk0 = ld_std_swz(sKtT, PC, 16 * ct, 0);
                const halfx8 fk1 = ld_std_swz(sKtT, PC, 16 * ct, 1);
                floatx4 wa[4];
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    // transposed product: lane holds W'[16R + ln][16ct + 4g .. +3]
                    wa[R] = mma16(fk0, ft[R][0], zero4());
                    if (R >= 2) wa[R] = mma16(fk1, ft[R][1], wa[R]);
                }
#pragma unroll
                for (int R = 0; R < 4; ++R) st_neg4(sW + (16 * R + ln) * PK + pcol(16 * ct + 4 * g4), wa[R]);
            }
            const halfx8 fx0 = ld_std_swz(sXT, PC, 16 * wave, 0);
            const halfx8 fx1 = ld_std_swz(sXT, PC, 16 * wave, 1);
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                D[R] = mma16(ft[R][0], fx0, zero4());
                if (R >= 2) D[R] = mma16(ft[R][1], fx1, D[R]);
            }
        } else {
            constexpr int NCT = DK / 16;  // column tiles of W'
            for (int ct = wave; ct < NCT; ct += 4) {
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    const int nk = (16 * R + 16 + KSTEP - 1) / KSTEP;
                    // transposed product: lane holds W'[16R + ln][16ct + 4g .. +3]
                    const floatx4 acc = mma_ls<true>(zero4(), sT, PC, 16 * R, sKtT, PC, 16 * ct, nk);
                    st_neg4(sW + (16 * R + ln) * PK + 16 * ct + 4 * g4, acc);
                }
            }
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const int nk = (16 * R + 16 + KSTEP - 1) / KSTEP;
                D[R] = mma_ls(zero4(), sT, PC, 16 * R, sXT, PC, 16 * wave, nk);
            }
        }
        if (pf) {
            load_part(cur, c0 + C, 3);
            load_part(cur, c0 + C, 4);
        }
        __syncthreads();

        // ---------------- 5. per-wave value side ---------------------------------
        // Sm = gamma_mid (.) S (rows = key channels) is the B operand of both
        // W' Sm (= W S) and Qt' Sm (= Qt S).
        if constexpr (CKPT) store_ckpt<DK>(args.ckpt, ck_slot + ci, H, h, DV, vcol0, Sacc);
        floatx4 Sm[NST];
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) Sm[t][jj] = Sacc[t][jj] * sGamM[16 * t + 4 * g4 + jj];
        RegB<Op, NST> SB;
        SB.build(Sm);
        RegB<Op, 4> DB;
        floatx4 O[4];  // O^T tiles: lane holds O[16R + ln][16 wave + 4g .. +3]
        floatx4 kd[NST];
        if constexpr (sizeof(Op) == 2) {
            constexpr int NM = NST / 2;
            // Delta = U - W S and the Qt S part of O: independent accumulators
            halfx8 fw[4][NM], fq[4][NM];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    fw[R][m] = ld_std(sW, PK, 16 * R, m);
                    if (!NOQ) fq[R][m] = ld_std(sQ2, PK, 16 * R, m);
                }
#pragma unroll
            for (int R = 0; R < 4; ++R) O[R] = zero4();
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    D[R] = mma16(fw[R][m], SB.f[m], D[R]);
                    if (!NOQ) O[R] = mma16(SB.f[m], fq[R][m], O[R]);
                }
            DB.build(D);
            halfx8 fp[4][2], fk[NST][2];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    if (!NOQ && m <= (R >> 1)) fp[R][m] = ld_std(sP, PC, 16 * R, m);
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int m = 0; m < 2; ++m) fk[t][m] = ld_std_swz(sKhT, PC, 16 * t, m);
#pragma unroll
            for (int t = 0; t < NST; ++t) kd[t] = zero4();
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int R = 0; R < 4; ++R)
                    if (!NOQ && m <= (R >> 1)) O[R] = mma16(DB.f[m], fp[R][m], O[R]);  // + P Delta
#pragma unroll
                for (int t = 0; t < NST; ++t) kd[t] = mma16(fk[t][m], DB.f[m], kd[t]);  // Kh'^T Delta
            }
        } else {
#pragma unroll
            for (int R = 0; R < 4; ++R) D[R] = mma_lr(D[R], sW, PK, 16 * R, 0, SB, NST);  // U - W S
            DB.build(D);
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                if (NOQ) continue;
                O[R] = mma_rl(zero4(), SB, NST, sQ2, PK, 16 * R);                        // Qt S
                O[R] = mma_rl(O[R], DB, R + 1, sP, PC, 16 * R);                          // + P Delta
            }
#pragma unroll
            for (int t = 0; t < NST; ++t) kd[t] = mma_lrs(zero4(), sKhT, PC, 16 * t, DB, 4);
        }
        // S <- gamma_C (.) S + (gamma_C/gamma_mid) (.) (Kh'^T Delta)
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 16 * t + 4 * g4 + jj;
                Sacc[t][jj] = Sacc[t][jj] * sGamC[i] + kd[t][jj] * sGamR[i];
            }
        if (!NOQ) {
#pragma unroll
            for (int R = 0; R < 4; ++R)
                *reinterpret_cast<floatx4*>(sO + (16 * R + ln) * PO + 16 * wave + 4 * g4) = O[R];
        }
        __syncthreads();
        if (!NOQ) {
            const int r = tid >> 2;
            const int cb = (tid & 3) * 16;
            if (r < clen) {
                Out* dst = o + (size_t)(row0 + c0 + r) * vstride + (size_t)h * DV + slab * SV + cb;
                const float* src = sO + r * PO + cb;
#pragma unroll
                for (int e = 0; e < 16; e += 4) store4(dst + e, src[e], src[e + 1], src[e + 2], src[e + 3]);
            }
        }
        // the next chunk's first LDS writes follow its first barrier
    }
    if (nchunks > 0 && s_bad) {
        init_state();
        token_serial_redo<In, Out, DK>(Sacc, args, args.gates == GATES_GDN,
                                       args.gates != GATES_FULL, NOQ, mslab, row0, len, h,
                                       vcol0, CKPT ? args.ckpt : nullptr, ck_slot);
    }
    if (CKPT && seg == nseg_n - 1) store_ckpt<DK>(args.ckpt, ck_final, H, h, DV, vcol0, Sacc);

    if (SUMMARY) {
        // columns [0, dv) of the map are H, [dv, dv + dk) are M
        const int W2 = DV + DK;
        float* sp = args.maps + ((size_t)pair * nseg + seg) * DK * W2 + slab * SV + 16 * wave + ln;
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) sp[(size_t)(16 * t + 4 * g4 + j) * W2] = Sacc[t][j];
    } else if (args.S_T && seg == nseg_n - 1) {
        float* sp = args.S_T + (size_t)pair * DK * DV + vcol0 + ln;
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) sp[(size_t)(16 * t + 4 * g4 + j) * DV] = Sacc[t][j];
    }
}

// ===========================================================================
// bf16 inputs: wave-specialised forward, pipelined over chunks
// ===========================================================================
// A workgroup of 8 waves owns one (sequence, head, 64-column value slab).
// Waves 0-3 (value waves) keep the fp32 state slab in registers, 16 value
// columns each; waves 4-7 (key waves) keep the raw inputs of the next chunk.
// Every chunk c runs two barrier-separated steps:
//   M. value waves: the state step of chunk c; key waves: decay products and
//      operand tiles of chunk c+1, then the loads of chunk c+2.  Each SIMD
//      runs one wave of each kind, so the value wave's MFMA and LDS reads
//      overlap the key wave's VALU work;
//   2. A (strictly lower blocks), the inverses T_ii = (I + A_ii)^-1 of its
//      16x16 diagonal blocks, and P of chunk c+1 (all waves).
// The state step never forms T = (I + A)^-1: with Z = X - Kt' Sm (Sm =
// gamma_mid (.) S), Delta = U - W S = T Z is the solution of
// (I + A) Delta = Z, found per wave for its 16 columns by block forward
// substitution, Delta_i = T_ii (Z_i - sum_{j<i} A_ij Delta_j).  Then
// O = Qt' Sm + P Delta and S <- gamma_C (.) S + (gamma_C/gamma_mid) (.) Kh'^T Delta.
// Tiles of chunk c that the state step reads while chunk c+1's are built
// (Kt', Qt', Kh'^T, X and the decay vectors) are double-buffered.  X is read
// along tokens with the LDS transpose read (ds_read_b64_tr_b16), and so is
// Kh'^T along channels for A and P, so each of them is stored once.
constexpr int WS_THREADS = 512;

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i & 3) of the 4-element row that lane 4e + (i >> 2) addressed, as its
// element e.
__device__ __forceinline__ halfx4 ld_tr(const _Float16* p) {
    const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
    return __builtin_bit_cast(halfx4, v);
}
__device__ __forceinline__ halfx8 cat8(halfx4 lo, halfx4 hi) {
    halfx8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}
// 16x16x32 fragment of a token-major [k][*] tile taken along its columns:
// lane (n, g) = (l & 15, l >> 4) receives rows k0 + 8g .. k0 + 8g + 7 of
// column n of a 16-column tile stored as four runs of four contiguous
// elements, run a at element offset c0 + rs * a.
__device__ __forceinline__ halfx8 tr8(const _Float16* tile, int pitch, int k0, int c0, int rs,
                                      int l) {
    const int j = l & 15;
    const _Float16* p = tile + (k0 + 8 * (l >> 4) + (j >> 2)) * pitch + c0 + rs * (j & 3);
    return cat8(ld_tr(p), ld_tr(p + 4 * pitch));
}
// As tr8 for the swizzled [channel][token] tile Kh'^T read along tokens 16S ..
// 16S + 15 (columns in permuted order), rows in the permuted contraction
// order {32m + 4g .. +3, 32m + 16 + 4g .. +3} of the fp16 operand tiles.
// Row 32m + 16h + x (x < 16) has swizzle key 2m + h, so the swizzled element
// offset of run a is 4(S & 1) + 32((S >> 1) ^ (m >> 1)) + 8(a ^ ((2m + h) & 3)):
// four per-lane bases (one per value of (2m + h) & 3) serve every (m, S).
struct KhtTrBases {
    const _Float16* p[4];
};
__device__ __forceinline__ KhtTrBases kht_tr_bases(const _Float16* tile, int pitch, int l) {
    const int j = l & 15;
    const _Float16* row = tile + (4 * (l >> 4) + (j >> 2)) * pitch;
    KhtTrBases b;
#pragma unroll
    for (int u = 0; u < 4; ++u) b.p[u] = row + 8 * ((j & 3) ^ u);
    return b;
}
// Kh' rows 16S .. 16S+15 (tokens), channels 32m .. 32m+31, from the Kh'^T
// tile (swz_kh): channel rows 32m + x have key 2m, rows 32m + 16 + x key
// 2m + 1, so the 8-column block of the lane's 4 tokens is XORed with m & 3
// in both reads and the 32-column half flips in the second
__device__ __forceinline__ halfx8 tr8_kht(const KhtTrBases& b, int pitch, int m, int S) {
    const int c0 = 32 * (S >> 1) + 4 * (S & 1);
    return cat8(ld_tr(b.p[m & 3] + 32 * m * pitch + c0),
                ld_tr(b.p[m & 3] + (32 * m + 16) * pitch + (c0 ^ 32)));
}

// A and P tiles of one chunk over 8 waves.  Value wave W computes the
// diagonal A tile (W, W), returned in registers in both orientations for the
// block inverse that follows, and the diagonal P tile (W, W), which shares
// its Kh' fragments; key waves take the 6 off-diagonal A tiles and the 6
// off-diagonal P tiles, three each, grouped so that they share fragments.
template <int W, int J>
__device__ __forceinline__ constexpr ApJob ws_job() {
    // A00 P00 | A11 P11 | A22 P22 | A33 P33 |
    // A10 A20 A30 | A21 A31 A32 | P10 P20 P30 | P21 P31 P32
    constexpr ApJob t[8][3] = {
        {{false, 0, 0}, {true, 0, 0}, {false, 0, 0}},
        {{false, 1, 1}, {true, 1, 1}, {false, 0, 0}},
        {{false, 2, 2}, {true, 2, 2}, {false, 0, 0}},
        {{false, 3, 3}, {true, 3, 3}, {false, 0, 0}},
        {{false, 1, 0}, {false, 2, 0}, {false, 3, 0}},
        {{false, 2, 1}, {false, 3, 1}, {false, 3, 2}},
        {{true, 1, 0}, {true, 2, 0}, {true, 3, 0}},
        {{true, 2, 1}, {true, 3, 1}, {true, 3, 2}}};
    return t[W][J];
}

template <int DK, int PK, int PKH, int PC, int W, bool WITH_P>
__device__ __forceinline__ void ws_ap_tiles(const _Float16* sKt, const _Float16* sKhT,
                                            const _Float16* sQ, _Float16* sP, _Float16* sA,
                                            floatx4& N, floatx4& Nt, int l) {
    constexpr bool DIAG = W < 4;
    constexpr int NJ = DIAG ? 2 : 3;
    const int g4 = l >> 4, ln = l & 15;
    constexpr ApJob jobs[3] = {ws_job<W, 0>(), ws_job<W, 1>(), ws_job<W, 2>()};
    constexpr bool skip_all = !WITH_P && jobs[0].isP;  // key waves 6, 7 without P
    if constexpr (skip_all) return;
    floatx4 acc[NJ];
    floatx4 accN = zero4();
#pragma unroll
    for (int jn = 0; jn < NJ; ++jn) acc[jn] = zero4();
    const KhtTrBases kb = kht_tr_bases(sKhT, PKH, l);
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
        halfx8 fa[NJ], fb[NJ];
#pragma unroll
        for (int jn = 0; jn < NJ; ++jn) {
            if (!WITH_P && jobs[jn].isP) continue;
            fa[jn] = ld_std_kq(jobs[jn].isP ? sQ : sKt, PK, jobs[jn].R, s, l);
            fb[jn] = tr8_kht(kb, PKH, s, jobs[jn].S);
        }
        // transposed products: lane holds row 16R + (l&15), columns 16S + 4g .. 4g+3
#pragma unroll
        for (int jn = 0; jn < NJ; ++jn)
            if (WITH_P || !jobs[jn].isP) acc[jn] = mma16(fb[jn], fa[jn], acc[jn]);
        if constexpr (DIAG) accN = mma16(fa[0], fb[0], accN);
    }
    constexpr int J0 = DIAG ? 1 : 0;
    if constexpr (DIAG) {
        // N[4g+j][ln] in accN, N^T[4g+j][ln] = N[ln][4g+j] in acc[0]
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            N[j] = (4 * g4 + j > ln) ? accN[j] : 0.f;
            Nt[j] = (ln > 4 * g4 + j) ? acc[0][j] : 0.f;
        }
    }
#pragma unroll
    for (int jn = J0; jn < NJ; ++jn) {
        if (!WITH_P && jobs[jn].isP) continue;
        const int r = 16 * jobs[jn].R + ln;
        floatx4 x = acc[jn];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 16 * jobs[jn].S + 4 * g4 + j;
            if (jobs[jn].isP ? (r < c) : (r <= c)) x[j] = 0.f;
        }
        if (jobs[jn].isP) st4(sP + r * PC + pcol(16 * jobs[jn].S + 4 * g4), x);
        else st4(sA + r * PC + 16 * jobs[jn].S + 4 * g4, x);
    }
}

template <typename Out, int DK, int MODE, int GM, int NSUB>
__global__ __launch_bounds__(WS_THREADS, 1) void fwd_ws_kernel(FwdArgs args) {
    using In = bf16_t;
    using Op = _Float16;
    const In* __restrict__ q = static_cast<const In*>(args.q);
    const In* __restrict__ k = static_cast<const In*>(args.k);
    const In* __restrict__ v = static_cast<const In*>(args.v);
    const In* __restrict__ alpha = static_cast<const In*>(args.alpha);
    const In* __restrict__ b = static_cast<const In*>(args.b);
    const In* __restrict__ w = static_cast<const In*>(args.w);
    Out* __restrict__ o = static_cast<Out*>(args.o);
    const int H = args.H, DV = args.DV, T = args.T;
    constexpr bool SUMMARY = MODE == MODE_SUMMARY;
    constexpr bool CKPT = MODE == MODE_CKPT;   // see fwd_kernel
    constexpr bool NOQ = SUMMARY || CKPT;
    // gates with one value per (token, head), [rows, H], broadcast over the
    // channels: alpha (GDN form), b and w (KDA and GDN forms)
    constexpr bool APH = GM == GATES_GDN;
    constexpr bool BPH = GM != GATES_FULL;
    constexpr int C = FWD_C;
    constexpr int SV = FWD_SV;
    constexpr int PK = DK + 16;    // pitch of the [C][DK] tiles (swz_kq)
    constexpr int PKH = C + 16;    // pitch of the [DK][C] tile Kh'^T (swz_kh)
    constexpr int PC = C + 8;      // pitch of the [C][C] tiles
    constexpr int PT = 24;         // pitch of the 16 x 16 diagonal blocks of T
    constexpr int PX = SV + 16;    // pitch of X: the transpose read of 4 rows x 16 columns is conflict-free
    constexpr int NST = DK / 16;   // state tiles per value wave
    // Key wave w takes channel half w & 1 and row half w >> 1 of a chunk:
    // NCGH 8-channel groups x 32 rows, so that one load instruction reads
    // whole 128-byte lines (dk = 128).  Relative to the chunk midpoint the two
    // row halves are independent: the first needs only products up to the
    // midpoint, the second only products after it.
    constexpr int NCGH = DK / 16;      // 8-channel groups per key wave
    constexpr int NRG = 64 / NCGH;     // row groups per key wave
    constexpr int RPTK = 32 / NRG;     // consecutive rows per key thread
    constexpr int NDR = NRG / 4;       // DPP rows holding one channel group (2 or 4)
    // raw input registers of the key waves: q, k, b, alpha, RPTK rows each
    constexpr int RQ = 0, RK = RPTK, RB = 2 * RPTK, RA = 3 * RPTK;

    // ---- workgroup -> (pair, segment, slab); slabs of one unit share an XCD ----
    // NSUB == 1: one workgroup per (unit, slab).  NSUB > 1 (segmented
    // plans): one workgroup per unit whose value waves take every slab in
    // turn, sub-slab sb = slab sb, so the key side of a chunk is built once
    // for all of them.
    const int nsl = args.nslab + (SUMMARY ? args.nslab_m : 0);
    const int nsub = NSUB > 1 ? nsl : 1;
    // the summary pass splits its sub-slabs between the roles: the value
    // waves take the first nsub_v (the value slabs first), the key waves the
    // rest (columns of M, which have no X), after their own tile work
    constexpr bool KV = SUMMARY && NSUB > 1;
    const int nsub_v = KV ? (nsub + 1) / 2 : nsub;
    const int nseg = args.nseg;
    const int unit = work_unit(args.num_pairs * nseg, NSUB > 1 ? 1 : nsl, args.order, args.H);
    if (unit < 0) return;
    const int slab = NSUB > 1 ? 0 : (blockIdx.x >> 3) % nsl;
    const int pair = unit / nseg;
    const int seg = unit - pair * nseg;
    auto slab_of = [&](int sb) { return NSUB > 1 ? sb : slab; };
    // a column block of M (X = 0)
    auto is_m = [&](int sb) { return SUMMARY && slab_of(sb) >= args.nslab; };
    // sub-slabs with X (the value slabs) come first: NSUB_H of them at most
    constexpr int NSUB_H = NSUB > 1 ? 2 : 1;
    const int nsub_h = NSUB > 1 ? args.nslab : 1;
    const int n = pair / H;
    const int h = pair - n * H;
    int64_t row0, len;
    int nseg_n;   // segments of this sequence
    seg_rows(args, n, seg, row0, len, nseg_n);
    if (seg >= nseg_n) return;                   // a packed sequence shorter than nseg slots
    if (SUMMARY && seg == nseg_n - 1) return;    // the last segment's map is never used

    // LDS regions (bytes); the first five are double-buffered by chunk parity
    constexpr int TK = C * PK * 2;    // [C][DK] tile
    constexpr int TT = DK * PKH * 2;  // [DK][C] tile
    constexpr int TX = C * PX * 2;    // [C][SV] tile
    constexpr int TC = C * PC * 2;    // [C][C] tile
    constexpr int OFF_KT = 0;                     // Kt'
    constexpr int OFF_KHT = OFF_KT + 2 * TK;      // Kh'^T
    constexpr int OFF_Q = OFF_KHT + 2 * TT;       // Qt'
    constexpr int OFF_X = OFF_Q + 2 * TK;         // X = w (.) v, token-major
    constexpr int OFF_G = OFF_X + 2 * TX;         // gamma_mid, gamma_C/gamma_mid
    constexpr int OFF_P = OFF_G + 2 * 2 * DK * 4; // P = tril(Qt' Kh'^T)
    constexpr int OFF_A = OFF_P + TC;             // A (strictly lower 16x16 blocks)
    constexpr int OFF_T = OFF_A + TC;             // T_ii = (I + A_ii)^-1, [4][16][PT]
    constexpr int LDS_BYTES = OFF_T + 4 * 16 * PT * 2;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __align__(16) unsigned char smem[LDS_BYTES];
    Op* const sKt0 = reinterpret_cast<Op*>(smem + OFF_KT);
    Op* const sKhT0 = reinterpret_cast<Op*>(smem + OFF_KHT);
    Op* const sQ0 = reinterpret_cast<Op*>(smem + OFF_Q);
    Op* const sX0 = reinterpret_cast<Op*>(smem + OFF_X);
    float* const sG0 = reinterpret_cast<float*>(smem + OFF_G);
    Op* const sP = reinterpret_cast<Op*>(smem + OFF_P);
    Op* const sA = reinterpret_cast<Op*>(smem + OFF_A);
    Op* const sT = reinterpret_cast<Op*>(smem + OFF_T);
    auto kt_buf = [&](int bb) { return sKt0 + bb * (TK / 2); };
    auto kht_buf = [&](int bb) { return sKhT0 + bb * (TT / 2); };
    auto q_buf = [&](int bb) { return sQ0 + bb * (TK / 2); };
    // X: double-buffered by chunk parity (NSUB == 1), or one buffer per value
    // sub-slab, written between a chunk's two barriers (NSUB > 1)
    auto x_buf = [&](int bb, int sb) { return sX0 + (NSUB > 1 ? sb : bb) * (TX / 2); };
    auto g_buf = [&](int bb) { return sG0 + bb * 2 * DK; };  // [gamma_mid | gamma_C/gamma_mid]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool VW = wave < 4;
    const int kwave = wave - 4;
    // Every step re-derives the lane index from a value the compiler cannot
    // see through, so that LDS and global addresses are formed where they are
    // used rather than held in registers across the chunk loop.
    // Key-wave thread layout: rows 32 krh + rgk*RPTK .. +RPTK-1 of its row
    // half, channels 8cg .. 8cg+7 of its channel half (kw_rgk, kw_cgl below);
    // value-wave layout of v, w and X: rows 16 wave + rv, 16 wave + 8 + rv,
    // slab columns 8cv .. 8cv+7.
    auto lane_ix = [&]() {
        int x = tid & 63;
        asm volatile("" : "+v"(x));
        return x;
    };
    // value waves: first state column of sub-slab sb
    auto vcol_of = [&](int sb) { return slab_of(sb) * SV + 16 * (wave & 3); };
    const size_t kstride = (size_t)H * DK;
    const size_t vstride = (size_t)H * DV;

    // upper-triangle tiles of P, which the P Delta product reads, stay zero:
    // every chunk rewrites only the lower tiles
    for (int e = tid; e < C * PC; e += WS_THREADS) sP[e] = (Op)0.f;
    // Set when some chunk's decay leaves the fp16 range of the
    // midpoint-referenced factors (see key_prep): each key wave collects its
    // chunks' verdicts in kbad and writes the flag before the last barrier.
    // The chunk loops run to the end regardless (same barriers, values then
    // discarded); after the last barrier the value waves redo the sequence
    // (segment) token by token.
    __shared__ int s_bad;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    uint64_t kbad = 0;
    // checkpoint mode: slot of this segment's first chunk, and of the
    // sequence's final state
    int64_t ck_slot = 0, ck_final = 0;
    if constexpr (CKPT) {
        const int64_t s0 = ckpt_slot0(args.cu_seqlens, T, n);
        ck_slot = s0 + (int64_t)seg * args.seg_chunks;
        const int64_t Ln = args.cu_seqlens ? (int64_t)args.cu_seqlens[n + 1] - args.cu_seqlens[n]
                                           : (int64_t)T;
        ck_final = s0 + (Ln + C - 1) / C;
    }
    // Value waves: running max of |x| over every value they convert to an
    // fp16 operand (X, Sm = gamma_mid (.) S, Delta, T_ii).  Above 2^15 (fp16
    // ends at 65504) the sequence (segment) goes to the token-serial path too.
    float vmax = 0.f;

    // Each role runs its own copy of the chunk loop, so that no loop-carried
    // register is shared between the roles: the value waves carry the state
    // tiles and one chunk's raw v, w; the key waves one chunk's raw q, k, b,
    // alpha (in flight while the previous chunk is computed).
    floatx4 ST[NSUB][NST];  // value waves: state rows 16t + 4g + j, column 16 wave + ln
    floatx4 VR[NSUB_H][4];  // value waves: raw v (rows m = 0, 1), raw w (2 + m)
    floatx4 KR[4 * RPTK];   // key waves
    const int64_t nchunks = (len + C - 1) / C;
    auto clen_of = [&](int64_t ci) { return (int)((len - ci * C) < C ? (len - ci * C) : C); };

    // ---- raw loads through buffer descriptors: one per tensor and chunk,
    // based at the chunk's first row of this head and sized to the chunk's
    // rows that lie inside the sequence (segment).  Rows past the end fall
    // outside the descriptor's range and read as zero; every later use of
    // such a row is masked.  The lane's offset is a 32-bit byte offset. ----
    auto chunk_rows = [&](int64_t cstart) {
        const int64_t rem = len - cstart;
        return (uint32_t)(rem <= 0 ? 0 : rem < C ? rem : C);
    };
    const uint32_t krow_bytes = (uint32_t)kstride * 2;
    const uint32_t vrow_bytes = (uint32_t)vstride * 2;
    struct KwSrc {
        __amdgpu_buffer_rsrc_t r[4];   // q, k, b, alpha
        uint32_t voff;                 // the lane's first row and channel group, bytes
        uint32_t soff;                 // the lane's first row in a per-(token, head) gate, bytes
    };
    const uint32_t grow_bytes = (uint32_t)H * 2;   // row pitch of a per-(token, head) gate
    // key-wave lane layout: row group (l >> 2) % NRG; channel group l & 3,
    // plus 4 for lanes 32 .. 63 when dk = 128
    auto kw_cgl = [&](int l) { return NCGH == 8 ? ((l & 3) | ((l >> 5) << 2)) : (l & 3); };
    auto kw_rgk = [&](int l) { return (l >> 2) & (NRG - 1); };
    const int kch = kwave & 1, krh = kwave >> 1;   // channel half, row half
    auto kw_ofs = [&](int64_t cstart, int l) {
        const int cg = kch * NCGH + kw_cgl(l), rgk = kw_rgk(l);
        const size_t e0 = (size_t)(row0 + cstart) * kstride + (size_t)h * DK;
        const uint32_t nb = chunk_rows(cstart) * krow_bytes;
        KwSrc o;
        o.r[0] = buf_rsrc(q + e0, nb);
        o.r[1] = buf_rsrc(k + e0, nb);
        const size_t g0 = (size_t)(row0 + cstart) * H + h;
        const uint32_t gb = chunk_rows(cstart) * grow_bytes;
        o.r[2] = BPH ? buf_rsrc(b + g0, gb) : buf_rsrc(b + e0, nb);
        o.r[3] = APH ? buf_rsrc(alpha + g0, gb) : buf_rsrc(alpha + e0, nb);
        o.voff = (uint32_t)(32 * krh + rgk * RPTK) * krow_bytes + 16u * (uint32_t)cg;
        o.soff = (uint32_t)(32 * krh + rgk * RPTK) * grow_bytes;
        return o;
    };
    // part 0..3 = q, k, b, alpha; row m of the thread's RPTK rows
    auto load_kw = [&](const KwSrc& o, int part, int m) {
        if (NOQ && part == 0) return;
        const int rr = part == 0 ? RQ : part == 1 ? RK : part == 2 ? RB : RA;
        if ((BPH && part == 2) || (APH && part == 3))
            KR[rr + m] = buf_ld2(o.r[part], o.soff + (uint32_t)m * grow_bytes);
        else
            KR[rr + m] = buf_ld16(o.r[part], o.voff + (uint32_t)m * krow_bytes);
    };
    auto load_vw = [&](int64_t cstart, int sb) {   // value waves, value sub-slab sb
        if (is_m(sb)) return;
        const int l = lane_ix();
        const int cv = l & 7, rv = l >> 3;
        const size_t e0 = (size_t)(row0 + cstart) * vstride + (size_t)h * DV + slab_of(sb) * SV;
        const uint32_t nb = chunk_rows(cstart) * vrow_bytes;
        const __amdgpu_buffer_rsrc_t rv_ = buf_rsrc(v + e0, nb);
        const __amdgpu_buffer_rsrc_t rw_ =
            BPH ? buf_rsrc(w + (size_t)(row0 + cstart) * H + h, chunk_rows(cstart) * grow_bytes)
                : buf_rsrc(w + e0, nb);
        const uint32_t voff = (uint32_t)(16 * wave + rv) * vrow_bytes + 16u * (uint32_t)cv;
        const uint32_t woff = (uint32_t)(16 * wave + rv) * grow_bytes;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            VR[sb][m] = buf_ld16_nt(rv_, voff + (uint32_t)(8 * m) * vrow_bytes);
            VR[sb][2 + m] = BPH ? buf_ld2(rw_, woff + (uint32_t)(8 * m) * grow_bytes)
                                : buf_ld16_nt(rw_, voff + (uint32_t)(8 * m) * vrow_bytes);
        }
    };
    // Declares a raw register overwritten once its widened values x exist:
    // the reload that follows then reuses the register, with no copy of the
    // old value kept for a later widening.
    auto retire = [&](floatx4& raw, const float (&x)[8]) {
        asm volatile("" : "+v"(raw) : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]),
                     "v"(x[5]), "v"(x[6]), "v"(x[7]));
    };
    auto widen = [&](const floatx4& src, float (&x)[8]) {
        const u16x8 u = __builtin_bit_cast(u16x8, src);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = bf16_to_f32(u[i]);
    };
    // a gate register: 8 channels, or (PH) one per-(token, head) value broadcast
    auto widen_gate = [&](auto ph_tag, const floatx4& src, float (&x)[8]) {
        if constexpr (decltype(ph_tag)::value) {
            const float g = bf16_to_f32((uint16_t)__float_as_uint(src[0]));
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = g;
        } else {
            widen(src, x);
        }
    };

    // ---- key waves, step 1: decay products and operand tiles of a chunk ----
    // Each raw register is reloaded with the chunk next_cstart as soon as its
    // value has been used (alpha after the scan, q, k, b row by row), so the
    // loads have most of a chunk period to arrive.
    auto key_prep = [&](auto full_tag, int clen, int bb, bool load_next, int64_t next_cstart) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int l = lane_ix();
        const int cg = kch * NCGH + kw_cgl(l), rgk = kw_rgk(l);
        const int rbase = 32 * krh + rgk * RPTK;   // the thread's first row
        Op* const sKt = kt_buf(bb);
        Op* const sKhT = kht_buf(bb);
        Op* const sQ = q_buf(bb);
        float* const sGam = g_buf(bb);
        float gp[RPTK][8];  // alpha, then the inclusive in-chunk product
#pragma unroll
        for (int m = 0; m < RPTK; ++m) {
            const bool ok = FULL || rbase + m < clen;
            widen_gate(std::integral_constant<bool, APH>{}, KR[RA + m], gp[m]);
#pragma unroll
            for (int i = 0; i < 8; ++i) gp[m][i] = ok ? gp[m][i] : 1.f;
        }
        float al[RPTK][8];    // the alphas (1 for absent rows), kept for the reciprocal chain below
#pragma unroll
        for (int m = 1; m < RPTK; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i) al[m][i] = gp[m][i];
        const KwSrc nofs = kw_ofs(next_cstart, l);
        if (load_next) {
#pragma unroll
            for (int m = 0; m < RPTK; ++m) {
                retire(KR[RA + m], gp[m]);
                load_kw(nofs, 3, m);
            }
        }
#pragma unroll
        for (int m = 1; m < RPTK; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i) gp[m][i] *= gp[m - 1][i];
        // pre: product of alpha over the half's rows before the thread's first
        // row, divided by gamma_mid in the first half (whose rows reach the
        // midpoint from below); tot: product over the whole half, i.e.
        // gamma_mid (first half) or gamma_C/gamma_mid (second half)
        float pre[8], tot[8];
        {
            // the NRG row groups of a channel group lie 4 lanes apart in NDR
            // consecutive 16-lane rows: inclusive scan inside each row, row
            // totals by a rotate-and-multiply butterfly, then across rows by
            // lane-swapping the totals between rows
            float inc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) inc[i] = tot[i] = gp[RPTK - 1][i];
            dpp_shr_mul8<4>(inc);
            dpp_shr_mul8<8>(inc);
            dpp_ror_mul8<4>(tot);
            dpp_ror_mul8<8>(tot);
            const int drow = l >> 4;   // DPP row of the lane
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // ev / od: the totals of the even and odd row of the lane's pair
                const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(tot[i]),
                                                                 __float_as_uint(tot[i]), false, false);
                const float ev = __uint_as_float(pr[0]), od = __uint_as_float(pr[1]);
                float e = (drow & 1) ? ev : 1.f;   // the earlier rows of this channel group
                if constexpr (NDR == 2) {
                    tot[i] = ev * od;
                } else {
                    const float pair = ev * od;
                    const auto ph = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair),
                                                                     __float_as_uint(pair), false, false);
                    const float lo = __uint_as_float(ph[0]), hi = __uint_as_float(ph[1]);
                    tot[i] = lo * hi;
                    e = (drow & 2) ? lo * e : e;
                }
                pre[i] = e;
            }
            // times the earlier row groups of the same 16-lane row
            dpp_shr_mul8_into<4>(inc, pre);
            if (krh == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) pre[i] *= __builtin_amdgcn_rcpf(tot[i]);
            }
        }
        // smallest half-chunk decay of the lane's channels (checked below)
        float mn = tot[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mn = fminf(mn, tot[i]);
        if (rgk == 0) {
            float4* d = reinterpret_cast<float4*>(sGam + krh * DK + 8 * cg);
            d[0] = make_float4(tot[0], tot[1], tot[2], tot[3]);
            d[1] = make_float4(tot[4], tot[5], tot[6], tot[7]);
        }
        // operand tiles relative to the chunk midpoint:
        //   Kt' = b k gamma_r/gamma_mid, Kh' = k gamma_mid/gamma_r, Qt' = q gamma_r/gamma_mid
        // 1/(gamma_r/gamma_mid) for the thread's RPTK rows from one reciprocal:
        // the last row's, times the alphas of the later rows (rows walked
        // from the last to the first)
        float tKh[8][RPTK];
        float e1i[8];
        float mx = 0.f;   // max |q|, |k| over the lane's rows and channels
#pragma unroll
        for (int i = 0; i < 8; ++i) e1i[i] = __builtin_amdgcn_rcpf(gp[RPTK - 1][i] * pre[i]);
#pragma unroll
        for (int m = RPTK - 1; m >= 0; --m) {
            const int r = rbase + m;
            if (m < RPTK - 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) e1i[i] *= al[m + 1][i];   // alpha of row m + 1
            }
            float gq[8], gk[8], gb[8];
            if (!NOQ) widen(KR[RQ + m], gq);
            else {
#pragma unroll
                for (int i = 0; i < 8; ++i) gq[i] = 0.f;
            }
            widen(KR[RK + m], gk);
            widen_gate(std::integral_constant<bool, BPH>{}, KR[RB + m], gb);
            if (load_next) {
                if (!NOQ) retire(KR[RQ + m], gq);
                retire(KR[RK + m], gk);
                retire(KR[RB + m], gb);
                load_kw(nofs, 0, m);
                load_kw(nofs, 1, m);
                load_kw(nofs, 2, m);
            }
            const bool ok = FULL || r < clen;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                gq[i] = ok ? gq[i] : 0.f;
                gk[i] = ok ? gk[i] : 0.f;
                mx = fmaxf(fmaxf(mx, fabsf(gq[i])), fabsf(gk[i]));   // v_max3_f32
            }
            float a1[8], a3[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e1 = gp[m][i] * pre[i];   // gamma_r / gamma_mid
                a1[i] = (gb[i] * gk[i]) * e1;
                a3[i] = gq[i] * e1;
                tKh[i][m] = gk[i] * e1i[i];
            }
            st_row8kq(sKt, PK, r, 8 * cg, a1);
            if (!NOQ) st_row8kq(sQ, PK, r, 8 * cg, a3);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 8 * cg + i;
            st_col<RPTK>(sKhT + row * PKH + swz_kh(row, pcol(rbase)), tKh[i]);
        }
        // fp16 range of this chunk's key-side operands.  The tiles are |q|,
        // |k| (b <= 1) times factors of at most 1/tot, and the entries of A
        // and P are sums of dk products of two such entries with factors of
        // at most 1.  They stay within 2^15 while the half-chunk decay is
        // at least 2^-14 in every channel, |q|, |k| <= 16 and
        // |q|, |k| <= 2^15 tot.  Otherwise (or on a non-finite value) the
        // whole sequence (segment) goes to the token-serial path.
        kbad |= __builtin_amdgcn_ballot_w64(!(mn >= 0x1p-14f && mx <= fminf(16.f, 0x1p15f * mn)));
    };
    // value waves: -X = -(w (.) v) of a chunk into sX (0 for absent rows and M
    // slabs); stored negated, so the state step's Y = Kt' Sm - X starts from
    // the tile as it is
    auto value_prep = [&](auto full_tag, int clen, int bb, int sb) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int l = lane_ix();
        const int cv = l & 7, rv = l >> 3;
        Op* const sX = x_buf(bb, sb);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int r = 16 * wave + 8 * m + rv;
            const bool ok = !is_m(sb) && (FULL || r < clen);
            float vv[8], ww[8], xv[8];
            widen(VR[sb][m], vv);
            widen_gate(std::integral_constant<bool, BPH>{}, VR[sb][2 + m], ww);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xv[i] = ok ? -(ww[i] * vv[i]) : 0.f;   // -X: the state step starts from it
                vmax = fmaxf(vmax, fabsf(xv[i]));
            }
            st_row8(sX + r * PX + 8 * cv, xv);
        }
    };

    // ---- step 2 for one chunk (its tiles built by key_prep) ----
    auto step2 = [&](int bb) {
        const int l = lane_ix();
        const int g4 = l >> 4, ln = l & 15;
        const Op* const sKt = kt_buf(bb);
        const Op* const sKhT = kht_buf(bb);
        const Op* const sQ = q_buf(bb);
        floatx4 N = zero4(), Nt = zero4();
        switch (wave) {
            case 0: ws_ap_tiles<DK, PK, PKH, PC, 0, !NOQ>(sKt, sKhT, sQ, sP, sA, N, Nt, l); break;
            case 1: ws_ap_tiles<DK, PK, PKH, PC, 1, !NOQ>(sKt, sKhT, sQ, sP, sA, N, Nt, l); break;
            case 2: ws_ap_tiles<DK, PK, PKH, PC, 2, !NOQ>(sKt, sKhT, sQ, sP, sA, N, Nt, l); break;
            case 3: ws_ap_tiles<DK, PK, PKH, PC, 3, !NOQ>(sKt, sKhT, sQ, sP, sA, N, Nt, l); break;
            case 4: ws_ap_tiles<DK, PK, PKH, PC, 4, !NOQ>(sKt, sKhT, sQ, sP, sA, N, Nt, l); break;
            case 5: ws_ap_tiles<DK, PK, PKH, PC, 5, !NOQ>(sKt, sKhT, sQ, sP, sA, N, Nt, l); break;
            case 6: ws_ap_tiles<DK, PK, PKH, PC, 6, !NOQ>(sKt, sKhT, sQ, sP, sA, N, Nt, l); break;
            default: ws_ap_tiles<DK, PK, PKH, PC, 7, !NOQ>(sKt, sKhT, sQ, sP, sA, N, Nt, l); break;
        }
        if (VW) {
            const floatx4 Tii = diag_block_inverse<Op>(N, Nt, l);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                sT[(16 * wave + 4 * g4 + jj) * PT + ln] = (Op)Tii[jj];
                vmax = fmaxf(vmax, fabsf(Tii[jj]));
            }
        }
        __syncthreads();
    };

    // ---- value waves, step M of one chunk, front: Delta (returned as the B
    // operand DB of the state update) and O ----
    auto value_step = [&](auto full_tag, int64_t c0, int clen, int bb, int sb,
                          floatx4 (&STs)[NST], RegB<Op, 4>& DB) {
        constexpr bool FULL = decltype(full_tag)::value;
        // Scheduling hint (interleave MFMA with LDS reads), measured: the
        // per-head gate forms take 4-5% less time with it, the full form 4%
        // more, so only the former use it.
        if constexpr (GM != GATES_FULL) __builtin_amdgcn_iglp_opt(0);
        const int l = lane_ix();
        const int g4 = l >> 4, ln = l & 15;
        const Op* const sKt = kt_buf(bb);
        const Op* const sKhT = kht_buf(bb);
        const Op* const sQ = q_buf(bb);
        const Op* const sX = x_buf(bb, sb);
        const float* const sGam = g_buf(bb);
        if constexpr (CKPT) store_ckpt<DK>(args.ckpt, ck_slot + c0 / C, H, h, DV, vcol_of(sb), STs);
        // Sm = gamma_mid (.) S (kept in ST for the rest of the step) is the B
        // operand of both Kt' Sm and Qt' Sm (= Qt S)
        RegB<Op, NST> SB;
#pragma unroll
        for (int t = 0; t < NST; ++t) {
            const float4 gm = *reinterpret_cast<const float4*>(sGam + 16 * t + 4 * g4);
            STs[t][0] *= gm.x;
            STs[t][1] *= gm.y;
            STs[t][2] *= gm.z;
            STs[t][3] *= gm.w;
            const int m = t >> 1, hf = 4 * (t & 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                SB.f[m][hf + j] = (Op)STs[t][j];
                vmax = fmaxf(vmax, fabsf(STs[t][j]));
            }
        }
        constexpr int NM = NST / 2;
        // Y = Kt' Sm - X (= -Z, Z = X - Kt' Sm): the accumulators start from
        // the -X tile, read in the accumulator layout (lane holds -X[16R + 4g +
        // j][16 (wave & 3) + ln] of the sub-slab) through the transpose read.  O^T
        // tiles: lane holds O[16R + ln][16 (wave & 3) + 4g .. +3]
        floatx4 Y[4], O[4];
        // a column block of M has X = 0 (and no X buffer)
        const bool mcols = is_m(sb);
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            O[R] = zero4();
            if (mcols) {
                Y[R] = zero4();
                continue;
            }
            const halfx4 x = ld_tr(sX + (16 * R + 4 * g4 + (ln >> 2)) * PX + 16 * (wave & 3) + 4 * (ln & 3));
#pragma unroll
            for (int j = 0; j < 4; ++j) Y[R][j] = (float)x[j];   // the tile holds -X
        }
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            halfx8 fk[NM], fq[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                fk[m] = ld_std_kq(sKt, PK, R, m, l);
                if (!NOQ) fq[m] = ld_std_kq(sQ, PK, R, m, l);
            }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                Y[R] = mma16(fk[m], SB.f[m], Y[R]);
                if (!NOQ) O[R] = mma16(SB.f[m], fq[m], O[R]);
            }
        }
        // (I + A) D = Y by block forward substitution over 16-token blocks:
        // D = -Delta
        floatx4 D[4];
        D[0] = blk_mma<Op>(zero4(), sT, PT, 0, 0, Y[0], l);
#pragma unroll
        for (int i = 1; i < 4; ++i) {
            floatx4 acc = zero4();
#pragma unroll
            for (int j = 0; j < i; ++j) acc = blk_mma<Op>(acc, sA, PC, 16 * i, 16 * j, D[j], l);
            floatx4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = Y[i][e] - acc[e];
            D[i] = blk_mma<Op>(zero4(), sT + 16 * i * PT, PT, 0, 0, r, l);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) vmax = fmaxf(vmax, fabsf(D[i][e]));
        DB.build_neg(D);   // Delta
        if (!NOQ) {
            halfx8 fp[4][2];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    if (m <= (R >> 1)) fp[R][m] = ld_std(sP, PC, 16 * R, m, l);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int R = 0; R < 4; ++R)
                    if (m <= (R >> 1)) O[R] = mma16(DB.f[m], fp[R][m], O[R]);  // + P Delta
            // O straight from registers: 4 consecutive columns of one row per
            // lane, through a descriptor sized to the chunk's rows in the
            // sequence (rows past the end are dropped by its range check)
            const uint32_t orow = (uint32_t)vstride * (uint32_t)sizeof(Out);
            const __amdgpu_buffer_rsrc_t ors =
                buf_rsrc(o + (size_t)(row0 + c0) * vstride + (size_t)h * DV + vcol_of(sb),
                         (uint32_t)(FULL ? C : clen) * orow);
            const uint32_t oofs = (uint32_t)ln * orow + (uint32_t)(4 * g4 * sizeof(Out));
#pragma unroll
            for (int R = 0; R < 4; ++R) buf_st4(ors, oofs + (uint32_t)(16 * R) * orow, O[R], o);
        }
    };
    // ---- value waves, step M of one chunk, back: the state update
    // S <- gamma_C (.) S + (gamma_C/gamma_mid) (.) (Kh'^T Delta)
    //    = (gamma_C/gamma_mid) (.) (Sm + Kh'^T Delta)   (ST holds Sm) ----
    auto value_update = [&](int bb, floatx4 (&STs)[NST], const RegB<Op, 4>& DB) {
        // Scheduling hint (interleave MFMA with LDS reads): measured 2% less
        // time for the full form and 1% for the KDA form.
        __builtin_amdgcn_iglp_opt(0);
        const int l = lane_ix();
        const int g4 = l >> 4, ln = l & 15;
        const Op* const sKhT = kht_buf(bb);
        const float* const sGam = g_buf(bb);
        // Kh'^T row 16t + ln (swz_kh, key t): its 16-byte block 32m + 8g
        // sits at 32(m ^ (t & 1)) + 8(g ^ ((t >> 1) & 3)); four per-lane bases
        const Op* kb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kb[u] = sKhT + ln * PKH + 8 * (g4 ^ u);
#pragma unroll
        for (int t = 0; t < NST; ++t) {
            const Op* pr = kb[(t >> 1) & 3] + 16 * t * PKH;
            const int hi = t & 1;
            const halfx8 fk0 = *reinterpret_cast<const halfx8*>(pr + 32 * hi);
            const halfx8 fk1 = *reinterpret_cast<const halfx8*>(pr + 32 * (1 ^ hi));
            floatx4 kd = mma16(fk0, DB.f[0], STs[t]);
            kd = mma16(fk1, DB.f[1], kd);
            const float4 gr = *reinterpret_cast<const float4*>(sGam + DK + 16 * t + 4 * g4);
            STs[t][0] = kd[0] * gr.x;
            STs[t][1] = kd[1] * gr.y;
            STs[t][2] = kd[2] * gr.z;
            STs[t][3] = kd[3] * gr.w;
        }
    };

    auto init_state = [&](int sb, floatx4 (&STs)[NST]) {
        const int l = tid & 63, g4 = l >> 4, ln = l & 15;
        const float* sp = nullptr;
        if (!SUMMARY) {
            // segmented: every start, S0's too, from the combine pass (see fwd_kernel)
            if (nseg == 1)
                sp = args.S0 ? args.S0 + (size_t)pair * DK * DV + vcol_of(sb) + ln : nullptr;
            else sp = args.starts + ((size_t)pair * nseg + seg) * DK * DV + vcol_of(sb) + ln;
        }
        if (sp) {
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) STs[t][j] = sp[(size_t)(16 * t + 4 * g4 + j) * DV];
        } else if (is_m(sb)) {
            // identity columns: M starts as I
            const int col = (slab_of(sb) - args.nslab) * SV + 16 * (wave & 3) + ln;
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) STs[t][j] = (16 * t + 4 * g4 + j == col) ? 1.f : 0.f;
        } else {
#pragma unroll
            for (int t = 0; t < NST; ++t) STs[t] = zero4();
        }
    };
    // after the last barrier: the token-serial redo (when flagged) and the
    // final stores of sub-slab sb
    auto finish_sub = [&](int sb) {
        if (nchunks > 0 && s_bad) {
            init_state(sb, ST[sb]);
            token_serial_redo<In, Out, DK>(ST[sb], args, APH, BPH, NOQ, is_m(sb), row0, len, h,
                                           vcol_of(sb), CKPT ? args.ckpt : nullptr, ck_slot);
        }
        if (CKPT && seg == nseg_n - 1)
            store_ckpt<DK>(args.ckpt, ck_final, H, h, DV, vcol_of(sb), ST[sb]);
        const int l = tid & 63, g4 = l >> 4, ln = l & 15;
        if (SUMMARY) {
            // columns [0, dv) of the map are H, [dv, dv + dk) are M
            const int W2 = DV + DK;
            float* sp = args.maps + ((size_t)pair * nseg + seg) * DK * W2 + vcol_of(sb) + ln;
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) sp[(size_t)(16 * t + 4 * g4 + j) * W2] = ST[sb][t][j];
        } else if (args.S_T && seg == nseg_n - 1) {
            float* sp = args.S_T + (size_t)pair * DK * DV + vcol_of(sb) + ln;
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) sp[(size_t)(16 * t + 4 * g4 + j) * DV] = ST[sb][t][j];
        }
    };
    // the state step of chunk ci on the sub-slabs sb in [lo, hi)
    auto state_steps = [&](int64_t ci, int lo, int hi) {
        const int bb = (int)(ci & 1);
        const int cc = clen_of(ci);
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
            if (sb >= lo && sb < hi) {
                RegB<Op, 4> DB;
                if (cc == C) value_step(std::true_type{}, ci * C, C, bb, sb, ST[sb], DB);
                else value_step(std::false_type{}, ci * C, cc, bb, sb, ST[sb], DB);
                value_update(bb, ST[sb], DB);
            }
        }
    };

    if (VW) {
        // ---- value waves ----
        // X of chunk ci into the buffer bb (NSUB == 1) or the sub-slab
        // buffers (NSUB > 1), then the loads of chunk ci + 1
        auto prep_x = [&](int64_t ci, int bb) {
#pragma unroll
            for (int sb = 0; sb < NSUB_H; ++sb) {
                if (sb < nsub_h) {
                    const int cn = clen_of(ci);
                    if (cn == C) value_prep(std::true_type{}, C, bb, sb);
                    else value_prep(std::false_type{}, cn, bb, sb);
                    if (ci + 1 < nchunks) load_vw((ci + 1) * C, sb);
                }
            }
        };
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb)
            if (sb < nsub_v) init_state(sb, ST[sb]);
#pragma unroll
        for (int sb = 0; sb < NSUB_H; ++sb)
#pragma unroll
            for (int m = 0; m < 4; ++m) VR[sb][m] = zero4();
        if (nchunks > 0) {
#pragma unroll
            for (int sb = 0; sb < NSUB_H; ++sb)
                if (sb < nsub_h) load_vw(0, sb);
            prep_x(0, 0);
            __syncthreads();
            step2(0);
            for (int64_t ci = 0; ci < nchunks; ++ci) {
                const int bb = (int)(ci & 1);
                const bool more = ci + 1 < nchunks;
                // NSUB == 1: X of chunk c+1 first (its loads landed long
                // ago), then the loads of chunk c+2, then the state step of
                // chunk c.  NSUB > 1: X of chunk c+1 after the barrier below.
                if (NSUB == 1 && more) prep_x(ci + 1, bb ^ 1);
                state_steps(ci, 0, nsub_v);
                // the value waves' verdict joins the key waves' before the
                // last barrier
                if (!more && __builtin_amdgcn_ballot_w64(!(vmax <= 0x1p15f)) != 0 &&
                    lane_ix() == 0)
                    s_bad = 1;
                __syncthreads();
                if (NSUB > 1 && more) prep_x(ci + 1, 0);
                if (more) step2(bb ^ 1);
            }
        }
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb)
            if (sb < nsub_v) finish_sub(sb);
    } else if (nchunks > 0) {
        // ---- key waves ----
        // Only the last chunk can be partial, so the loop body prepares full
        // chunks only (one code path: the reloaded registers need no copies
        // that would wait for the loads); the last chunk is peeled.  The
        // barrier count matches the value waves' loop.
#pragma unroll
        for (int m = 0; m < 4 * RPTK; ++m) KR[m] = zero4();
        if constexpr (KV) {
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb)
                if (sb >= nsub_v && sb < nsub) init_state(sb, ST[sb]);
        }
        {
            const int cl = clen_of(0);
            const KwSrc o0 = kw_ofs(0, lane_ix());
#pragma unroll
            for (int part = 0; part < 4; ++part)
#pragma unroll
                for (int m = 0; m < RPTK; ++m) load_kw(o0, part, m);
            if (cl == C) key_prep(std::true_type{}, cl, 0, nchunks > 1, (int64_t)C);
            else key_prep(std::false_type{}, cl, 0, nchunks > 1, (int64_t)C);
        }
        __syncthreads();
        step2(0);
        int64_t ci = 0;
        for (; ci + 2 < nchunks; ++ci) {   // chunk ci+1 is full
            const int bb = (int)(ci & 1);
            key_prep(std::true_type{}, C, bb ^ 1, true, (ci + 2) * C);
            if constexpr (KV) state_steps(ci, nsub_v, nsub);
            __syncthreads();
            step2(bb ^ 1);
        }
        if (ci + 1 < nchunks) {            // the last chunk
            const int bb = (int)(ci & 1);
            const int cl = clen_of(ci + 1);
            if (cl == C) key_prep(std::true_type{}, cl, bb ^ 1, false, (int64_t)0);
            else key_prep(std::false_type{}, cl, bb ^ 1, false, (int64_t)0);
            if constexpr (KV) state_steps(ci, nsub_v, nsub);
            __syncthreads();
            step2(bb ^ 1);
            ++ci;
        }
        if constexpr (KV) {
            state_steps(ci, nsub_v, nsub);   // the last chunk
            kbad |= __builtin_amdgcn_ballot_w64(!(vmax <= 0x1p15f));
        }
        if (kbad != 0 && lane_ix() == 0) s_bad = 1;
        __syncthreads();                   // the value waves' last state step
        if constexpr (KV) {
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb)
                if (sb >= nsub_v && sb < nsub) finish_sub(sb);
        }
    }
}

// ---------------------------------------------------------------------------
// length order of a packed batch (longest first; ties by index)
// ---------------------------------------------------------------------------
// Thread i counts the sequences that come before sequence i, reading the
// lengths through LDS 256 at a time, and writes order[rank] = i.
__global__ __launch_bounds__(256) void seq_order_kernel(const int32_t* __restrict__ cu, int N,
                                                        int32_t* __restrict__ order) {
    __shared__ int sl[256];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int li = i < N ? cu[i + 1] - cu[i] : 0;
    int rank = 0;
    for (int base = 0; base < N; base += 256) {
        const int jj = base + (int)threadIdx.x;
        sl[threadIdx.x] = jj < N ? cu[jj + 1] - cu[jj] : -1;
        __syncthreads();
        const int lim = min(256, N - base);
        for (int t = 0; t < lim; ++t) {
            const int lj = sl[t];
            rank += (lj > li) || (lj == li && base + t < i);
        }
        __syncthreads();
    }
    if (i < N) order[rank] = i;
}

// ---------------------------------------------------------------------------
// segment combine: start state of every segment from the composed maps
// ---------------------------------------------------------------------------
// For one (sequence, head) pair and 16 value columns: S_start[0] = S0 (or 0),
// S_start[g+1] = M_g S_start[g] + H_g, g = 0 .. nseg-2, in fp32.  One
// workgroup of DK/16 waves per (pair, 16-column block); wave w computes rows
// 16w .. 16w+15 of each product on v_mfma_f32_16x16x4f32, with H_g as the
// accumulator's start.  The current start state lives in LDS (the B
// operand, shared by the waves); each lane reads its A operand, a run of M_g
// rows, with float4 loads, and the next step's M and H are loaded during the
// current product.  Contraction step t = 4q + e of lane group g takes index
// 16q + 4g + e, the same permutation on both operands.
template <int DK>
__global__ __launch_bounds__(DK * 4) void seg_combine_kernel(const float* __restrict__ maps,
                                                             float* __restrict__ starts,
                                                             const float* __restrict__ S0,
                                                             int nseg, int DV, FwdArgs args) {
    constexpr int NQ = DK / 16;              // float4 runs of a lane's M row
    const int ncb = DV / 16;
    // the column blocks of one pair run on one XCD (workgroups are dealt to
    // the 8 XCDs round-robin), so each map is read from HBM once and from
    // that XCD's L2 by the other blocks
    const int jb = blockIdx.x >> 3;
    const int pair = (jb / ncb) * 8 + (blockIdx.x & 7);
    if (pair >= args.num_pairs) return;
    const int c0 = (jb % ncb) * 16;
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63;
    const int col = l & 15, g = l >> 4;
    const int W2 = DV + DK;
    int64_t row0_unused, len_unused;
    int nseg_n;   // this sequence's segments (slots nseg_n .. nseg-1 are unused)
    seg_rows(args, pair / args.H, 0, row0_unused, len_unused, nseg_n);
    // pitch 20: the four lane groups' rows (4 apart) fall in disjoint banks
    __shared__ float sS[DK][20];
    // segment 0 starts from S0: copied to its start slot, which the forward
    // pass reads (so that pass never reads S0, which S_T may overwrite)
    float* const st0 = starts + (size_t)pair * nseg * DK * DV;
    for (int e = tid; e < DK * 16; e += DK * 4) {
        const int i = e >> 4, c = e & 15;
        const float x = S0 ? S0[((size_t)pair * DK + i) * DV + c0 + c] : 0.f;
        sS[i][c] = x;
        st0[(size_t)i * DV + c0 + c] = x;
    }
    // two maps in registers, alternating: map gs + 2 is loaded as soon as
    // map gs has been multiplied, so each load has a whole step to land
    float4 amA[NQ], amB[NQ];   // M_g[16w + col][16q + 4g .. +3]
    floatx4 hmA, hmB;          // H_g[16w + 4g + j][c0 + col]
    auto load = [&](int gs, float4 (&am)[NQ], floatx4& hm) {
        const float* base = maps + ((size_t)pair * nseg + gs) * DK * W2;
        const float* mrow = base + (size_t)(16 * w + col) * W2 + DV + 4 * g;
#pragma unroll
        for (int q = 0; q < NQ; ++q) am[q] = *reinterpret_cast<const float4*>(mrow + 16 * q);
#pragma unroll
        for (int j = 0; j < 4; ++j) hm[j] = base[(size_t)(16 * w + 4 * g + j) * W2 + c0 + col];
    };
    // S_start[gs + 1] = M_gs S_start[gs] + H_gs, with sS holding S_start[gs]
    auto step = [&](int gs, float4 (&am)[NQ], const floatx4& hm) {
        floatx4 acc = hm;
        __syncthreads();   // sS holds S_start[gs]
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int k = 16 * q + 4 * g;
            acc = mma16(am[q].x, sS[k][col], acc);
            acc = mma16(am[q].y, sS[k + 1][col], acc);
            acc = mma16(am[q].z, sS[k + 2][col], acc);
            acc = mma16(am[q].w, sS[k + 3][col], acc);
        }
        floatx4 h2 = hm;
        if (gs + 3 < nseg_n) load(gs + 2, am, h2);
        __syncthreads();   // every wave has read S_start[gs]
        float* dst = starts + ((size_t)pair * nseg + gs + 1) * DK * DV;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = 16 * w + 4 * g + j;
            sS[i][col] = acc[j];
            dst[(size_t)i * DV + c0 + col] = acc[j];
        }
        return h2;
    };
    if (nseg_n > 1) load(0, amA, hmA);
    if (nseg_n > 2) load(1, amB, hmB);
    for (int gs = 0; gs + 1 < nseg_n; gs += 2) {
        hmA = step(gs, amA, hmA);
        if (gs + 2 < nseg_n) hmB = step(gs + 1, amB, hmB);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Segment plan: a batch with fewer (sequence, head, slab) workgroups than
// compute units splits each sequence into segments (summary, combine and
// forward passes), so that the serial chunk walk is shared by more CUs.  For
// a packed batch the host does not know the lengths: the segment length comes
// from the packed token count, and the kernels find each sequence's segment
// count on the device.
constexpr int FWD_TARGET_WGS = 256;   // MI355X compute units
constexpr int FWD_MIN_SEG_CHUNKS = 8;

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

FwdPlan plan_fwd(int B, int T, int H, int dk, int dv, int num_seqs, int in_dtype) {
    FwdPlan p;
    p.nslab = dv / FWD_SV;
    p.nslab_m = dk / FWD_SV;
    p.nseg = 1;
    p.seg_chunks = 0;
    p.maps_off = p.starts_off = 0;
    p.order = false;
    p.order_off = 0;
    p.workspace = 0;
    // workgroups per (pair, segment) of a segmented plan: the bf16 kernel
    // takes every slab in one workgroup, the fp32 kernel one per slab; the
    // token-serial forward (fp32 at dk = 128) takes the bf16 kernel's plan
    const bool serial = in_dtype == DT_F32 && dk == 128;
    const int64_t wpu = in_dtype == DT_BF16 || serial ? 1 : p.nslab;
    if (B == 1 && num_seqs > 1) {
        // a packed batch (with cu_seqlens): room for its length order (not
        // used by the token-serial forward)
        p.order = !serial;
        p.workspace = serial ? 0 : align256((size_t)num_seqs * sizeof(int32_t));
        // Few (sequence, head, slab) workgroups: segments of seg_chunks chunks,
        // sized from the packed token count so that all sequences' segments
        // together fill the compute units.  The host does not know the
        // lengths, so each sequence gets slots for the longest possible one
        // (T tokens); a workgroup past its own sequence's segments exits.
        const int64_t pairs = (int64_t)num_seqs * H;
        const int64_t nch = ((int64_t)T + FWD_C - 1) / FWD_C;
        if (pairs * p.nslab >= FWD_TARGET_WGS) return p;
        int64_t sc = nch * H * wpu / FWD_TARGET_WGS;
        if (sc < FWD_MIN_SEG_CHUNKS) sc = FWD_MIN_SEG_CHUNKS;
        const int64_t kmax = (nch + sc - 1) / sc;
        if (kmax <= 1) return p;
        p.nseg = (int)kmax;
        p.seg_chunks = (int)sc;
        p.maps_off = p.workspace;
        p.starts_off = p.maps_off + align256((size_t)pairs * kmax * dk * (dv + dk) * sizeof(float));
        p.workspace = p.starts_off + align256((size_t)pairs * kmax * dk * dv * sizeof(float));
        return p;
    }
    const int64_t pairs = (int64_t)B * H;
    const int64_t nchunks = ((int64_t)T + FWD_C - 1) / FWD_C;
    if (num_seqs != B || pairs <= 0 || pairs * p.nslab >= FWD_TARGET_WGS) return p;
    int64_t nseg = (FWD_TARGET_WGS + pairs * wpu - 1) / (pairs * wpu);
    if (nseg > nchunks / FWD_MIN_SEG_CHUNKS) nseg = nchunks / FWD_MIN_SEG_CHUNKS;
    if (nseg <= 1) return p;
    const int64_t seg_chunks = (nchunks + nseg - 1) / nseg;
    nseg = (nchunks + seg_chunks - 1) / seg_chunks;
    if (nseg <= 1) return p;
    p.nseg = (int)nseg;
    p.seg_chunks = (int)seg_chunks;
    p.maps_off = 0;
    p.starts_off = align256((size_t)pairs * nseg * dk * (dv + dk) * sizeof(float));
    p.workspace = p.starts_off + align256((size_t)pairs * nseg * dk * dv * sizeof(float));
    return p;
}

template <typename In, typename Out, int DK, int GM>
static hipError_t launch_fwd_t(const FwdPlan& plan, const FwdArgs& a0, void* workspace,
                               hipStream_t stream) {
    FwdArgs a = a0;
    const bool seg = plan.nseg > 1;
    a.nseg = seg ? plan.nseg : 1;
    a.seg_chunks = seg ? plan.seg_chunks : 0;
    a.nslab_m = plan.nslab_m;
    a.maps = seg ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.maps_off) : nullptr;
    a.starts = seg ? reinterpret_cast<const float*>(static_cast<char*>(workspace) + plan.starts_off)
                   : nullptr;
    a.order = nullptr;
    const int nseqs = a.num_pairs / a.H;
    if (a.cu_seqlens && plan.order && nseqs > 1 && !seg) {
        int32_t* ord = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + plan.order_off);
        hipLaunchKernelGGL(seq_order_kernel, dim3((unsigned)((nseqs + 255) / 256)), dim3(256), 0,
                           stream, a.cu_seqlens, nseqs, ord);
        a.order = ord;
    }
    const int units = a.num_pairs * a.nseg;
    const unsigned groups = (unsigned)((units + 7) / 8);
    constexpr bool WS = std::is_same<In, bf16_t>::value;  // fp16 operands: wave-specialised kernel
    // segmented plans: one wave-specialised workgroup per (pair, segment)
    // covers every slab (the summary pass's M slabs too)
    constexpr int NSUB_S = DK / FWD_SV + 2;   // dv / 64 + dk / 64 slabs at most
    if (seg) {
        if constexpr (WS)
            hipLaunchKernelGGL((fwd_ws_kernel<float, DK, MODE_SUMMARY, GM, NSUB_S>),
                               dim3(groups * 8), dim3(WS_THREADS), 0, stream, a);
        else
            hipLaunchKernelGGL((fwd_kernel<In, float, DK, MODE_SUMMARY>),
                               dim3(groups * 8 * (a.nslab + a.nslab_m)), dim3(FWD_THREADS), 0, stream, a);
        hipLaunchKernelGGL((seg_combine_kernel<DK>), dim3((unsigned)((a.num_pairs + 7) / 8 * 8 * (a.DV / 16))),
                           dim3(DK * 4), 0, stream, a.maps, const_cast<float*>(a.starts), a.S0, a.nseg,
                           a.DV, a);
    }
    if (a.ckpt) {
        // checkpoint mode of the backward: no outputs (instantiated for fp32 Out only)
        if constexpr (std::is_same<Out, float>::value) {
            if constexpr (WS) {
                if (seg)
                    hipLaunchKernelGGL((fwd_ws_kernel<float, DK, MODE_CKPT, GM, 2>),
                                       dim3(groups * 8), dim3(WS_THREADS), 0, stream, a);
                else
                    hipLaunchKernelGGL((fwd_ws_kernel<float, DK, MODE_CKPT, GM, 1>),
                                       dim3(groups * 8 * a.nslab), dim3(WS_THREADS), 0, stream, a);
            } else
                hipLaunchKernelGGL((fwd_kernel<In, float, DK, MODE_CKPT>),
                                   dim3(groups * 8 * a.nslab), dim3(FWD_THREADS), 0, stream, a);
        } else {
            return hipErrorInvalidValue;
        }
    } else if constexpr (WS) {
        if (seg)
            hipLaunchKernelGGL((fwd_ws_kernel<Out, DK, MODE_FWD, GM, 2>), dim3(groups * 8),
                               dim3(WS_THREADS), 0, stream, a);
        else
            hipLaunchKernelGGL((fwd_ws_kernel<Out, DK, MODE_FWD, GM, 1>), dim3(groups * 8 * a.nslab),
                               dim3(WS_THREADS), 0, stream, a);
    } else {
        hipLaunchKernelGGL((fwd_kernel<In, Out, DK, MODE_FWD>), dim3(groups * 8 * a.nslab),
                           dim3(FWD_THREADS), 0, stream, a);
    }
    return hipGetLastError();
}

template <typename In, typename Out, int GM>
static hipError_t launch_fwd_gm(const FwdPlan& plan, const FwdArgs& a, int dk, void* workspace,
                                hipStream_t stream) {
    // fp32 operand tiles for dk = 128 would need 253 KB of LDS (160 KB limit):
    // that case runs the token-serial forward instead
    if constexpr (sizeof(typename OpOf<In>::type) == 2) {
        if (dk == 128) return launch_fwd_t<In, Out, 128, GM>(plan, a, workspace, stream);
    }
    if (dk != 64) return hipErrorInvalidValue;
    return launch_fwd_t<In, Out, 64, GM>(plan, a, workspace, stream);
}

// The bf16 kernel is compiled per gate form; the fp32 kernel reads a.gates.
template <typename In, typename Out>
static hipError_t launch_fwd_dk(const FwdPlan& plan, const FwdArgs& a, int dk, void* workspace,
                                hipStream_t stream) {
    if constexpr (std::is_same<In, bf16_t>::value) {
        if (a.gates == GATES_KDA) return launch_fwd_gm<In, Out, GATES_KDA>(plan, a, dk, workspace, stream);
        if (a.gates == GATES_GDN) return launch_fwd_gm<In, Out, GATES_GDN>(plan, a, dk, workspace, stream);
    }
    return launch_fwd_gm<In, Out, GATES_FULL>(plan, a, dk, workspace, stream);
}

hipError_t launch_fwd_serial_plan(const FwdPlan& plan, const void* q, const void* k,
                                  const void* v, const void* alpha, const void* b, const void* w,
                                  int in_dtype, const float* S0, void* o, int out_dtype,
                                  float* S_T, const int32_t* cu_seqlens, int N, int T, int H,
                                  int dk, int dv, int gates, bool erase_rows, void* workspace,
                                  hipStream_t stream, float* ckpt) {
    if (plan.nseg <= 1)
        return launch_fwd_serial(q, k, v, alpha, b, w, in_dtype, S0, o, out_dtype, S_T,
                                 cu_seqlens, N, T, H, dk, dv, gates, erase_rows, stream, ckpt);
    float* maps = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.maps_off);
    float* starts = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.starts_off);
    hipError_t e = launch_fwd_serial(q, k, v, alpha, b, w, in_dtype, nullptr, nullptr, out_dtype,
                                     nullptr, cu_seqlens, N, T, H, dk, dv, gates, erase_rows,
                                     stream, nullptr, plan.nseg, plan.seg_chunks, 1, maps, nullptr);
    if (e != hipSuccess) return e;
    // the combine pass reads the sequences' segment counts like the kernels
    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.b = b; a.w = w;
    a.S0 = S0; a.o = o; a.S_T = S_T; a.cu_seqlens = cu_seqlens;
    a.num_pairs = N * H;
    a.nslab = plan.nslab;
    a.T = T; a.H = H; a.DV = dv;
    a.nseg = plan.nseg; a.seg_chunks = plan.seg_chunks; a.nslab_m = plan.nslab_m;
    a.maps = maps; a.starts = starts;
    a.order = nullptr;
    a.gates = gates;
    a.ckpt = nullptr;
    const dim3 cgrid((unsigned)((a.num_pairs + 7) / 8 * 8 * (dv / 16)));
    if (dk == 128)
        hipLaunchKernelGGL((seg_combine_kernel<128>), cgrid, dim3(128 * 4), 0, stream, maps, starts,
                           S0, plan.nseg, dv, a);
    else
        hipLaunchKernelGGL((seg_combine_kernel<64>), cgrid, dim3(64 * 4), 0, stream, maps, starts,
                           S0, plan.nseg, dv, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_fwd_serial(q, k, v, alpha, b, w, in_dtype, S0, o, out_dtype, S_T, cu_seqlens, N,
                             T, H, dk, dv, gates, erase_rows, stream, ckpt, plan.nseg,
                             plan.seg_chunks, 0, nullptr, starts);
}

hipError_t launch_fwd(const FwdPlan& plan, const void* q, const void* k, const void* v,
                      const void* alpha, const void* b, const void* w, int in_dtype,
                      const float* S0, void* o, int out_dtype, float* S_T,
                      const int32_t* cu_seqlens, int num_seqs, int B, int T, int H, int dk,
                      int dv, int gates, void* workspace, hipStream_t stream, float* ckpt) {
    const int N = cu_seqlens ? num_seqs : B;
    if (N == 0 || ((int64_t)B * T == 0 && S_T == nullptr && ckpt == nullptr))
        return hipSuccess;  // nothing to do
    if (in_dtype == DT_F32 && dk == 128)
        return launch_fwd_serial_plan(plan, q, k, v, alpha, b, w, in_dtype, S0, o, out_dtype,
                                      ckpt ? nullptr : S_T, cu_seqlens, N, T, H, dk, dv, gates,
                                      false, workspace, stream, ckpt);
    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.b = b; a.w = w;
    a.S0 = S0; a.o = o; a.S_T = S_T; a.cu_seqlens = cu_seqlens;
    a.num_pairs = N * H;
    a.nslab = plan.nslab;
    a.T = T; a.H = H; a.DV = dv;
    a.nseg = 1; a.seg_chunks = 0; a.nslab_m = 0; a.maps = nullptr; a.starts = nullptr;
    a.order = nullptr;
    a.gates = gates;
    a.ckpt = ckpt;
    if (ckpt) {
        if (in_dtype == DT_BF16) return launch_fwd_dk<bf16_t, float>(plan, a, dk, workspace, stream);
        return launch_fwd_dk<float, float>(plan, a, dk, workspace, stream);
    }
    if (in_dtype == DT_BF16) {
        if (out_dtype == DT_BF16) return launch_fwd_dk<bf16_t, bf16_t>(plan, a, dk, workspace, stream);
        return launch_fwd_dk<bf16_t, float>(plan, a, dk, workspace, stream);
    }
    return launch_fwd_dk<float, float>(plan, a, dk, workspace, stream);
}

}  // namespace gdn2
