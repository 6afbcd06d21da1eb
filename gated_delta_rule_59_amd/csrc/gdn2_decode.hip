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
// Work split: one workgroup of 512 threads per (sequence, head), covering all
// dv value columns of its state.  Thread t owns 4 consecutive columns (one
// float4) of dk / (2048 / dv) rows (8 at dk = dv = 128), so dv / 4 lanes
// cover one whole row and every state byte is loaded and stored exactly once.
// The token vectors are loaded before the state, by every thread (clamped
// indices, no branch), so their loads do not queue behind the workgroup's
// own state loads (64 KB at d = 128).  On N = 256, H = 16, d = 128 with fresh token vectors per step:
// 32-column slabs (four workgroups per (sequence, head), token loads after
// the state's) took 90.6 us per step; the same slabs with the token loads
// first 86.2 us; one workgroup of 256 threads per (sequence, head) 82.4 us,
// of 512 threads 80.8 us (of 1024 threads 80.5 us).
#include "gdn2_common.hpp"
#include "gdn2_internal.h"

namespace gdn2 {

constexpr int DEC_THREADS = 512;

template <typename In, typename Out, int DK, int DV, bool EA>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const In* __restrict__ alpha, const In* __restrict__ b, const In* __restrict__ w,
    float* __restrict__ S, Out* __restrict__ o, int gates, int npairs) {
    constexpr int CG = DV / 4;              // threads across a row (float4 each)
    constexpr int RG = DEC_THREADS / CG;    // row groups
    constexpr int RPT = DK / RG;            // rows per thread
    static_assert(CG <= 64 && RPT * RG == DK, "row layout");
    const int pair = blockIdx.x;   // n * H + h
    if (pair >= npairs) return;
    const int tid = threadIdx.x;
    const int c4 = tid % CG;
    const int rg = tid / CG;

    // sized for every thread: all threads load and store their token values
    // (the copies past DK or DV are never read), so nothing here branches and
    // the token loads are issued ahead of the state loads
    __shared__ float sq[DEC_THREADS], sk[DEC_THREADS], sa[DEC_THREADS], sbk[DEC_THREADS],
        sx[DEC_THREADS];
    __shared__ float sred[DEC_THREADS / 64][CG][8];
    __shared__ float sqk, sqbk;
    const size_t kb = (size_t)pair * DK;
    const size_t vb = (size_t)pair * DV;
    const int ti = tid & (DK - 1), tj = tid & (DV - 1);
    const float tk = load1(k + kb + ti);
    const float tq = load1(q + kb + ti);
    // a per-(token, head) gate ([N, H]) is broadcast over the channels
    const float ta = load1(alpha + (gates == GATES_GDN ? (size_t)pair : kb + ti));
    const float tb = load1(b + (gates != GATES_FULL ? (size_t)pair : kb + ti));
    const float tw = load1(w + (gates != GATES_FULL ? (size_t)pair : vb + tj));
    const float tv = load1(v + vb + tj);

    float* Sp = S + (size_t)pair * DK * DV + c4 * 4;
    // the state is read once: non-temporal loads (measured 1.3% less time
    // per step; non-temporal stores as well made it 10% slower)
    float4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const floatx4 x = __builtin_nontemporal_load(
            reinterpret_cast<const floatx4*>(Sp + (size_t)(rg + m * RG) * DV));
        s[m] = make_float4(x[0], x[1], x[2], x[3]);
    }
    sq[tid] = tq;
    sk[tid] = tk;
    sa[tid] = ta;
    sbk[tid] = tb * tk;
    sx[tid] = tw * tv;
    __syncthreads();
    if (tid < 64) {  // q . k (and q . (b k) for the erase-on-rows reading) by wave 0
        float acc = 0.f, acb = 0.f;
        for (int i = tid; i < DK; i += 64) {
            acc += sq[i] * sk[i];
            if (EA) acb += sq[i] * sbk[i];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            acc += __shfl_xor(acc, off);
            if (EA) acb += __shfl_xor(acb, off);
        }
        if (tid == 0) {
            sqk = acc;
            sqbk = acb;
        }
    }

    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
    // this thread's rows of k (and b (.) k) are kept in registers for the
    // update, so its state stores issue back to back with no LDS wait between
    // them (read per store from LDS, the stores trickled out one by one:
    // 90.0 against 81.8 us per step at N = 256, H = 16, d = 128)
    float kr[RPT], bkr[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        kr[m] = sk[i];
        bkr[m] = sbk[i];
        // the prediction is read with b (.) k, or with k when b gates the rows
        const float a = sa[i], bk = EA ? kr[m] : bkr[m], qi = sq[i];
        s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
        r0 += bk * s[m].x; r1 += bk * s[m].y; r2 += bk * s[m].z; r3 += bk * s[m].w;
        p0 += qi * s[m].x; p1 += qi * s[m].y; p2 += qi * s[m].z; p3 += qi * s[m].w;
    }
    // sum over the row groups of a wave (lanes c4, c4 + CG, ...)
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
    if constexpr (!EA) {
        float dl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) dl[j] = sx[c4 * 4 + j] - rr[j];

#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float ki = kr[m];
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
    } else {
        // b on the erased rows: S <- S' + k x^T - (b (.) k) r^T with r = S'^T k,
        // o = S'^T q + (q . k) x - (q . (b k)) r
        float xx[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xx[j] = sx[c4 * 4 + j];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float ki = kr[m], bki = bkr[m];
            float4 t;
            t.x = s[m].x + ki * xx[0] - bki * rr[0]; t.y = s[m].y + ki * xx[1] - bki * rr[1];
            t.z = s[m].z + ki * xx[2] - bki * rr[2]; t.w = s[m].w + ki * xx[3] - bki * rr[3];
            *reinterpret_cast<float4*>(Sp + (size_t)(rg + m * RG) * DV) = t;
        }
        if (rg == 0) {
            const float qk = sqk, qbk = sqbk;
            store4(o + vb + c4 * 4, pp[0] + qk * xx[0] - qbk * rr[0],
                   pp[1] + qk * xx[1] - qbk * rr[1], pp[2] + qk * xx[2] - qbk * rr[2],
                   pp[3] + qk * xx[3] - qbk * rr[3]);
        }
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

namespace {
// A token input as loaded (bf16 bits in the low half, or the fp32 value),
// widened only where it is used, SER_PF tokens later: widened at the load,
// behind the branch on the sequence end, it was waited for on the spot, and
// that wait (vmcnt) also covered the o stores issued before it.
__device__ __forceinline__ uint32_t ser_raw(const bf16_t* p) { return p->bits; }
__device__ __forceinline__ float ser_raw(const float* p) { return *p; }
__device__ __forceinline__ float ser_widen(uint32_t bits) { return __uint_as_float(bits << 16); }
__device__ __forceinline__ float ser_widen(float x) { return x; }
}  // namespace

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

// Segments (nseg > 1): a long sequence is split into segments of seg_chunks
// 64-token chunks, one wave per (pair, segment, 16 columns).  The summary
// pass (summary != 0) runs each segment but the last from a zero state for
// the dv columns and from the identity for dk more columns with no write
// (w (.) v = 0): the segment's affine state map S_end = M S_start + H, stored
// as maps[pair][seg][dk][dv + dk] = [H | M].  After the combine pass has
// chained the maps into starts[pair][seg][dk][dv] (S0 for segment 0), the
// forward pass runs every segment from its start.
struct SerSeg {
    int nseg, seg_chunks, summary;
    float* maps;
    const float* starts;
};

// SEG = false: one unsegmented pass (nseg == 1, no summary), compiled
// without the segment logic so that the token loop keeps the plain kernel's
// registers (the segment fields otherwise push scalar registers into VGPR
// lanes that the loop reads back every token).
template <typename In, typename Out, int DK, bool EA, bool SEG>
__global__ __launch_bounds__(64) void fwd_serial_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const In* __restrict__ alpha, const In* __restrict__ b, const In* __restrict__ w,
    const float* S0, Out* __restrict__ o, float* S_T, const int32_t* __restrict__ cu_seqlens,
    int T, int H, int DV, int gates, float* ckpt, SerSeg sg) {
    constexpr int RPL = DK / 64;   // key rows per lane
    const int ncb = DV / 16;
    // column blocks per (pair, segment): the summary pass adds dk / 16 of M
    const bool summary = SEG && sg.summary;
    const int nseg = SEG ? sg.nseg : 1;
    const int ncbt = summary ? ncb + DK / 16 : ncb;
    const int cb = (int)(blockIdx.x % (unsigned)ncbt);
    const int ps = (int)(blockIdx.x / (unsigned)ncbt);
    const int seg = SEG ? ps % nseg : 0, pair = SEG ? ps / nseg : ps;
    const bool mcol = summary && cb >= ncb;   // a column block of M
    const int c0 = (mcol ? cb - ncb : cb) * 16;
    const int n = pair / H, h = pair - n * H;
    int64_t start, L;
    if (cu_seqlens) {
        start = cu_seqlens[n];
        L = (int64_t)cu_seqlens[n + 1] - start;
    } else {
        start = (int64_t)n * T;
        L = T;
    }
    // the segment's rows (segments start at multiples of 64 tokens)
    int64_t row0 = start, len = L;
    int nseg_n = 1;
    if (SEG && nseg > 1) {
        const int64_t srows = (int64_t)sg.seg_chunks * 64;
        const int64_t nch = (L + 63) / 64;
        nseg_n = nch <= 0 ? 1 : (int)((nch + sg.seg_chunks - 1) / sg.seg_chunks);
        if (seg >= nseg_n) return;                  // a packed sequence with fewer segments
        if (summary && seg == nseg_n - 1) return;   // the last map is never used
        const int64_t s0 = (int64_t)seg * srows;
        row0 = start + s0;
        len = L - s0 < srows ? L - s0 : srows;
        if (len < 0) len = 0;
    }
    const bool last = seg == nseg_n - 1;
    const int l = threadIdx.x;
    const int cf = l >> 2;   // the column this lane holds after the reduce-scatter
    const size_t sbase = (size_t)pair * DK * DV + c0;

    // start state: zero or the identity's columns (summary), S0 (one
    // segment) or the segment's start from the combine pass
    float s[RPL][16];
    const float* src0 = nullptr;
    if (!summary)
        src0 = nseg > 1 ? sg.starts + ((size_t)pair * nseg + seg) * DK * DV + c0
                        : (S0 ? S0 + sbase : nullptr);
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const int row = l * RPL + i;
        const float* src = src0 ? src0 + (size_t)row * DV : nullptr;
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (src) x = *reinterpret_cast<const float4*>(src + j);
            s[i][j] = x.x; s[i][j + 1] = x.y; s[i][j + 2] = x.z; s[i][j + 3] = x.w;
        }
        if (SEG && mcol) {
#pragma unroll
            for (int j = 0; j < 16; ++j) s[i][j] = (row == c0 + j) ? 1.f : 0.f;
        }
    }

    // the inputs of one token for this lane: its key rows of alpha, b, q, k
    // and w, v of column c0 + cf (zero for a column block of M)
    using RawT = decltype(ser_raw(q));
    struct Tok { RawT a[RPL], bb[RPL], qq[RPL], kk[RPL], ww, vv; };
    // tokens past the end load the last token (in range, no branch); they
    // are never used
    auto fetch = [&](int64_t t0_, Tok& x) {
        const int64_t t = t0_ < len ? t0_ : len - 1;
        const size_t kr = ((size_t)(row0 + t) * H + h) * DK + (size_t)l * RPL;
        // a column block of M reads column 0 (in range) and zeroes it
        const size_t vr = ((size_t)(row0 + t) * H + h) * DV + (SEG && mcol ? 0 : c0 + cf);
        const size_t th = (size_t)(row0 + t) * H + h;   // a per-(token, head) gate
        const bool ga = gates == GATES_GDN, gbw = gates != GATES_FULL;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            x.a[i] = ser_raw(alpha + (ga ? th : kr + i));
            x.bb[i] = ser_raw(b + (gbw ? th : kr + i));
            x.qq[i] = ser_raw(q + kr + i);
            x.kk[i] = ser_raw(k + kr + i);
        }
        x.ww = ser_raw(w + (gbw ? th : vr));
        x.vv = ser_raw(v + vr);
    };
    Tok pf[SER_PF];
    if (len > 0)
#pragma unroll
        for (int u = 0; u < SER_PF; ++u) fetch(u, pf[u]);
    // backward checkpoints (o not written): the state before every 64th token
    // of the sequence and its final state, in slots ckpt_slot0(n) ..
    const int64_t ck0 =
        ckpt ? ckpt_slot0(cu_seqlens, T, n) + (SEG ? (int64_t)seg * sg.seg_chunks : 0) : 0;
    auto store_state = [&](float* base) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            float* dst = base + (size_t)(l * RPL + i) * DV;
#pragma unroll
            for (int j = 0; j < 16; j += 4)
                *reinterpret_cast<float4*>(dst + j) = make_float4(s[i][j], s[i][j + 1], s[i][j + 2], s[i][j + 3]);
        }
    };
    auto ck_ptr = [&](int64_t slot) { return ckpt + ((size_t)slot * H + h) * DK * DV + c0; };
    const bool write_o = !ckpt && !summary;

    // one token: t its index, u its prefetch slot (a constant in every
    // unrolled call)
    auto token = [&](const int64_t t, const int u) {
        // token t widened (a column block of M has no value term); the
        // empty asm keeps the widening (and the wait for these loads)
        // here, where the compiler had moved it to the end of the
        // previous group of SER_PF tokens, behind all of their loads
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            asm volatile("" : "+v"(pf[u].a[i]), "+v"(pf[u].bb[i]), "+v"(pf[u].qq[i]), "+v"(pf[u].kk[i]));
        asm volatile("" : "+v"(pf[u].ww), "+v"(pf[u].vv));
        struct { float a[RPL], bb[RPL], qq[RPL], kk[RPL], ww, vv; } x;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            x.a[i] = ser_widen(pf[u].a[i]);
            x.bb[i] = ser_widen(pf[u].bb[i]);
            x.qq[i] = ser_widen(pf[u].qq[i]);
            x.kk[i] = ser_widen(pf[u].kk[i]);
        }
        x.ww = SEG && mcol ? 0.f : ser_widen(pf[u].ww);
        x.vv = ser_widen(pf[u].vv);
        fetch(t + SER_PF, pf[u]);
        if (ckpt && (t & 63) == 0) store_state(ck_ptr(ck0 + t / 64));
        float r[16], p[16], qk = 0.f, qbk = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) { r[j] = 0.f; p[j] = 0.f; }
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const float bk = x.bb[i] * x.kk[i];
            const float rk = EA ? x.kk[i] : bk;   // the key that reads the prediction
            qk += x.qq[i] * x.kk[i];
            if (EA) qbk += x.qq[i] * bk;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                s[i][j] *= x.a[i];
                r[j] += rk * s[i][j];
                p[j] += x.qq[i] * s[i][j];
            }
        }
        const float rf = reduce_scatter16(r, l), pfc = reduce_scatter16(p, l);
        const float qkt = reduce_all(qk);
        const size_t oi = ((size_t)(row0 + t) * H + h) * DV + c0 + cf;
        if constexpr (!EA) {
            const float d = x.ww * x.vv - rf;   // delta of column cf
            if (write_o && (l & 3) == 0) store1(o + oi, pfc + qkt * d);
            float dl[16];
            all_gather16(d, l, dl);
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int j = 0; j < 16; ++j) s[i][j] += x.kk[i] * dl[j];
        } else {
            // b on the erased rows: S <- S' + k x^T - (b (.) k) r^T
            const float xc = x.ww * x.vv;
            const float qbkt = reduce_all(qbk);
            if (write_o && (l & 3) == 0) store1(o + oi, pfc + qkt * xc - qbkt * rf);
            float xl[16], rl[16];
            all_gather16(xc, l, xl);
            all_gather16(rf, l, rl);
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const float bk = x.bb[i] * x.kk[i];
#pragma unroll
                for (int j = 0; j < 16; ++j) s[i][j] += x.kk[i] * xl[j] - bk * rl[j];
            }
        }
    };
    // whole groups of SER_PF tokens with no branch between them, then the
    // last, partial group: with a branch out of the group after every token,
    // the joins at the loop's end needed copies of the prefetch registers,
    // and each copy waited for its loads (and the o stores before them)
    int64_t t0 = 0;
    for (; t0 + SER_PF <= len; t0 += SER_PF) {
#pragma unroll
        for (int u = 0; u < SER_PF; ++u) token(t0 + u, u);
    }
#pragma unroll
    for (int u = 0; u < SER_PF; ++u)
        if (t0 + u < len) token(t0 + u, u);
    if (summary) {
        // column c0 + j of H (dv columns) or of M (dk more)
        const int W2 = DV + DK;
        float* dst = sg.maps + ((size_t)pair * nseg + seg) * DK * W2 + (mcol ? DV : 0) + c0;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            float* d = dst + (size_t)(l * RPL + i) * W2;
#pragma unroll
            for (int j = 0; j < 16; j += 4)
                *reinterpret_cast<float4*>(d + j) = make_float4(s[i][j], s[i][j + 1], s[i][j + 2], s[i][j + 3]);
        }
        return;
    }
    if (S_T && last) store_state(S_T + sbase);
    if (ckpt && last) store_state(ckpt + ((size_t)(ckpt_slot0(cu_seqlens, T, n) + (L + 63) / 64) * H + h) * DK * DV + c0);
}

template <typename In, typename Out, bool EA>
static hipError_t launch_fwd_serial_t(const void* q, const void* k, const void* v,
                                      const void* alpha, const void* b, const void* w,
                                      const float* S0, void* o, float* S_T,
                                      const int32_t* cu_seqlens, int N, int T, int H, int dk,
                                      int dv, int gates, hipStream_t stream, float* ckpt,
                                      const SerSeg& sg) {
    const int ncbt = dv / 16 + (sg.summary ? dk / 16 : 0);
    const dim3 grid((unsigned)((size_t)N * H * sg.nseg * ncbt));
    const dim3 block(64);
#define GDN2_SER_ARGS                                                                          \
    static_cast<const In*>(q), static_cast<const In*>(k), static_cast<const In*>(v),           \
        static_cast<const In*>(alpha), static_cast<const In*>(b), static_cast<const In*>(w),   \
        S0, static_cast<Out*>(o), S_T, cu_seqlens, T, H, dv, gates, ckpt, sg
    if (sg.nseg > 1) {
        if (dk == 128)
            hipLaunchKernelGGL((fwd_serial_kernel<In, Out, 128, EA, true>), grid, block, 0, stream, GDN2_SER_ARGS);
        else
            hipLaunchKernelGGL((fwd_serial_kernel<In, Out, 64, EA, true>), grid, block, 0, stream, GDN2_SER_ARGS);
    } else {
        if (dk == 128)
            hipLaunchKernelGGL((fwd_serial_kernel<In, Out, 128, EA, false>), grid, block, 0, stream, GDN2_SER_ARGS);
        else
            hipLaunchKernelGGL((fwd_serial_kernel<In, Out, 64, EA, false>), grid, block, 0, stream, GDN2_SER_ARGS);
    }
#undef GDN2_SER_ARGS
    return hipGetLastError();
}

hipError_t launch_fwd_serial(const void* q, const void* k, const void* v, const void* alpha,
                             const void* b, const void* w, int in_dtype, const float* S0,
                             void* o, int out_dtype, float* S_T, const int32_t* cu_seqlens,
                             int N, int T, int H, int dk, int dv, int gates, bool erase_rows,
                             hipStream_t stream, float* ckpt, int nseg, int seg_chunks,
                             int summary, float* maps, const float* starts) {
    SerSeg sg;
    sg.nseg = nseg > 1 ? nseg : 1;
    sg.seg_chunks = nseg > 1 ? seg_chunks : 0;
    sg.summary = summary;
    sg.maps = maps;
    sg.starts = starts;
#define GDN2_SER_CALL(IN_, OUT_, EA_)                                                        \
    return launch_fwd_serial_t<IN_, OUT_, EA_>(q, k, v, alpha, b, w, S0, o, S_T, cu_seqlens, \
                                               N, T, H, dk, dv, gates, stream, ckpt, sg)
    if (in_dtype == DT_BF16) {
        if (out_dtype == DT_BF16) {
            if (erase_rows) GDN2_SER_CALL(bf16_t, bf16_t, true);
            GDN2_SER_CALL(bf16_t, bf16_t, false);
        }
        if (erase_rows) GDN2_SER_CALL(bf16_t, float, true);
        GDN2_SER_CALL(bf16_t, float, false);
    }
    if (erase_rows) GDN2_SER_CALL(float, float, true);
    GDN2_SER_CALL(float, float, false);
#undef GDN2_SER_CALL
}

template <typename In, typename Out, bool EA>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const void* alpha,
                                  const void* b, const void* w, float* S, void* o, int N, int H,
                                  int dk, int dv, int gates, hipStream_t stream) {
    const int npairs = N * H;
    const dim3 grid((unsigned)npairs);
    const dim3 block(DEC_THREADS);
#define GDN2_DEC_ARGS                                                                       \
    static_cast<const In*>(q), static_cast<const In*>(k), static_cast<const In*>(v),       \
        static_cast<const In*>(alpha), static_cast<const In*>(b), static_cast<const In*>(w), \
        S, static_cast<Out*>(o), gates, npairs
#define GDN2_DEC_LAUNCH(DK_, DV_) \
    hipLaunchKernelGGL((decode_kernel<In, Out, DK_, DV_, EA>), grid, block, 0, stream, GDN2_DEC_ARGS)
    if (dk == 128 && dv == 128) GDN2_DEC_LAUNCH(128, 128);
    else if (dk == 128) GDN2_DEC_LAUNCH(128, 64);
    else if (dv == 128) GDN2_DEC_LAUNCH(64, 128);
    else GDN2_DEC_LAUNCH(64, 64);
#undef GDN2_DEC_LAUNCH
#undef GDN2_DEC_ARGS
    return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* alpha,
                         const void* b, const void* w, int in_dtype, float* S, void* o,
                         int out_dtype, int N, int H, int dk, int dv, int gates,
                         hipStream_t stream, bool erase_rows) {
#define GDN2_DEC_CALL(IN_, OUT_, EA_) \
    return launch_decode_t<IN_, OUT_, EA_>(q, k, v, alpha, b, w, S, o, N, H, dk, dv, gates, stream)
    if (in_dtype == DT_BF16) {
        if (out_dtype == DT_BF16) {
            if (erase_rows) GDN2_DEC_CALL(bf16_t, bf16_t, true);
            GDN2_DEC_CALL(bf16_t, bf16_t, false);
        }
        if (erase_rows) GDN2_DEC_CALL(bf16_t, float, true);
        GDN2_DEC_CALL(bf16_t, float, false);
    }
    if (erase_rows) GDN2_DEC_CALL(float, float, true);
    GDN2_DEC_CALL(float, float, false);
#undef GDN2_DEC_CALL
}

}  // namespace gdn2
